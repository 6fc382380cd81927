// C ABI of the attention forward: argument validation, then kernel launch.
// Every check happens on the host before any HIP call, so an invalid call
// enqueues nothing and needs no device.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>

#include "ta03.h"
#include "ta03_internal.h"

namespace ta03 {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // 0: not queried yet
std::atomic<int> g_prefill_rows{0};
std::atomic<int> g_bwd_path{0};
}  // namespace

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
        n = 256;
    g_cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

int override_prefill_rows() { return g_prefill_rows.load(std::memory_order_relaxed); }
int override_bwd_path() { return g_bwd_path.load(std::memory_order_relaxed); }

}  // namespace ta03

namespace {

constexpr long long kMaxElems = 1ll << 31;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool head_dim_supported(int d) { return d == 64 || d == 128; }

// Shared validation and launch of attn_fwd_ex and attn_fwd_rope (rope_cs ==
// nullptr: no rotation).
int fwd_common(const float* q, long long q_stride, const float* k, long long k_stride,
               const float* v, long long v_stride, float* out, long long out_stride,
               float* lse, int q_base, int q_seq, int kv_len, int num_heads,
               int num_kv_heads, int head_dim, int mode, int start_pos, float scale,
               bool rope, const float* rope_cs, int rope_rows, hipStream_t stream,
               bool rope_keys = true) {
    if (num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0) return TA03_ERR_SHAPE;
    if (q_seq < 0 || kv_len < 0 || start_pos < 0 || q_base < 0) return TA03_ERR_SHAPE;
    if (mode != TA03_CAUSAL && mode != TA03_FULL && mode != TA03_CROSS) return TA03_ERR_SHAPE;
    if (mode != TA03_CAUSAL && start_pos != 0) return TA03_ERR_SHAPE;
    if (mode == TA03_CAUSAL && (long long)start_pos + q_base + q_seq > kv_len) return TA03_ERR_SHAPE;
    if (mode == TA03_FULL && (long long)q_base + q_seq > kv_len) return TA03_ERR_SHAPE;
    if (!std::isfinite(scale)) return TA03_ERR_SHAPE;
    if (!head_dim_supported(head_dim)) return TA03_ERR_UNSUPPORTED;
    const long long qd = (long long)num_heads * head_dim;
    const long long kvd = (long long)num_kv_heads * head_dim;
    if (q_stride < qd || out_stride < qd || k_stride < kvd || v_stride < kvd) return TA03_ERR_SHAPE;
    if (q_stride >= kMaxElems || out_stride >= kMaxElems || k_stride >= kMaxElems ||
        v_stride >= kMaxElems)
        return TA03_ERR_UNSUPPORTED;
    if (rope) {
        // Positions used: query rows start_pos + q_base .. + q_seq - 1, keys 0 .. kv_len - 1
        // (when the keys are turned here).
        const long long need = std::max((long long)start_pos + q_base + q_seq,
                                        rope_keys ? (long long)kv_len : 0ll);
        if (rope_rows < 0 || (q_seq > 0 && rope_rows < need)) return TA03_ERR_SHAPE;
        if ((long long)rope_rows * head_dim >= kMaxElems) return TA03_ERR_UNSUPPORTED;
    }
    if (q_seq == 0) return TA03_OK;
    if (q == nullptr || out == nullptr) return TA03_ERR_NULL;
    if (kv_len > 0 && (k == nullptr || v == nullptr)) return TA03_ERR_NULL;
    if (rope && rope_cs == nullptr) return TA03_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || !aligned16(k) || !aligned16(v) || !aligned16(lse) ||
        !aligned16(rope_cs) || (q_stride | k_stride | v_stride | out_stride) % 4 != 0)
        return TA03_ERR_ALIGN;

    ta03::PrefillShape s;
    s.q_seq = q_seq;
    s.kv_len = kv_len;
    s.num_heads = num_heads;
    s.num_kv_heads = num_kv_heads;
    s.head_dim = head_dim;
    s.causal = mode == TA03_CAUSAL ? 1 : 0;
    s.start_pos = start_pos + q_base;  // position of the first row handled
    s.scale = scale;
    s.q_stride = q_stride;
    s.k_stride = k_stride;
    s.v_stride = v_stride;
    s.out_stride = out_stride;
    s.rope_cs = rope ? rope_cs : nullptr;
    s.rope_keys = rope_keys;
    // Row q_base of the batch is row 0 of this launch.
    const float* qb = q + (size_t)q_base * (size_t)q_stride;
    float* ob = out + (size_t)q_base * (size_t)out_stride;
    float* lb = lse != nullptr ? lse + (size_t)q_base * (size_t)num_heads * 2 : nullptr;
    const hipError_t e = ta03::launch_prefill(qb, k, v, ob, lb, s, stream);
    return e == hipSuccess ? TA03_OK : TA03_ERR_HIP;
}

}  // namespace

extern "C" {

int attn_fwd_ex(const float* q, long long q_stride, const float* k, long long k_stride,
                const float* v, long long v_stride, float* out, long long out_stride,
                float* lse, int q_base, int q_seq, int kv_len, int num_heads,
                int num_kv_heads, int head_dim, int mode, int start_pos, float scale,
                hipStream_t stream) {
    return fwd_common(q, q_stride, k, k_stride, v, v_stride, out, out_stride, lse, q_base,
                      q_seq, kv_len, num_heads, num_kv_heads, head_dim, mode, start_pos, scale,
                      false, nullptr, 0, stream);
}

int attn_fwd_rope(const float* q, long long q_stride, const float* k, long long k_stride,
                  const float* v, long long v_stride, float* out, long long out_stride,
                  float* lse, int q_base, int q_seq, int kv_len, int num_heads,
                  int num_kv_heads, int head_dim, int mode, int start_pos, float scale,
                  const float* rope_cs, int rope_rows, hipStream_t stream) {
    return fwd_common(q, q_stride, k, k_stride, v, v_stride, out, out_stride, lse, q_base,
                      q_seq, kv_len, num_heads, num_kv_heads, head_dim, mode, start_pos, scale,
                      true, rope_cs, rope_rows, stream);
}

int attn_fwd_rope_q(const float* q, long long q_stride, const float* k, long long k_stride,
                    const float* v, long long v_stride, float* out, long long out_stride,
                    float* lse, int q_base, int q_seq, int kv_len, int num_heads,
                    int num_kv_heads, int head_dim, int mode, int start_pos, float scale,
                    const float* rope_cs, int rope_rows, hipStream_t stream) {
    return fwd_common(q, q_stride, k, k_stride, v, v_stride, out, out_stride, lse, q_base,
                      q_seq, kv_len, num_heads, num_kv_heads, head_dim, mode, start_pos, scale,
                      true, rope_cs, rope_rows, stream, false);
}

int attn_rope_apply(const float* x, long long x_stride, float* y, long long y_stride, int rows,
                    int heads, int head_dim, int pos0, const float* rope_cs, int rope_rows,
                    hipStream_t stream) {
    if (rows < 0 || heads < 1 || pos0 < 0 || head_dim < 8 || head_dim % 8 != 0)
        return TA03_ERR_SHAPE;
    const long long width = (long long)heads * head_dim;
    if (x_stride < width || y_stride < width) return TA03_ERR_SHAPE;
    if (rope_rows < 0 || (rows > 0 && (long long)rope_rows < (long long)pos0 + rows))
        return TA03_ERR_SHAPE;
    if (x_stride >= kMaxElems || y_stride >= kMaxElems || width >= kMaxElems ||
        (long long)rope_rows * head_dim >= kMaxElems)
        return TA03_ERR_UNSUPPORTED;
    if (rows == 0) return TA03_OK;
    if (x == nullptr || y == nullptr || rope_cs == nullptr) return TA03_ERR_NULL;
    if (!aligned16(x) || !aligned16(y) || !aligned16(rope_cs) || (x_stride | y_stride) % 4 != 0)
        return TA03_ERR_ALIGN;
    // In place (y == x, the same stride) or into memory that x does not cover.
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(x), y0 = reinterpret_cast<uintptr_t>(y);
    const uintptr_t x1 = x0 + (uintptr_t)(((long long)(rows - 1) * x_stride + width) * 4);
    const uintptr_t y1 = y0 + (uintptr_t)(((long long)(rows - 1) * y_stride + width) * 4);
    const bool same = x0 == y0 && x_stride == y_stride;
    if (!same && x0 < y1 && y0 < x1) return TA03_ERR_SHAPE;
    const hipError_t e = ta03::launch_rope_apply(x, x_stride, y, y_stride, rows, heads, head_dim,
                                                 pos0, rope_cs, stream);
    return e == hipSuccess ? TA03_OK : TA03_ERR_HIP;
}

size_t attn_bwd_workspace_bytes(int q_seq, int num_heads) {
    if (q_seq < 0 || num_heads < 1) return 0;
    const size_t n = 2 * (size_t)q_seq * (size_t)num_heads * sizeof(float);
    return (n + 255) / 256 * 256;
}

size_t attn_bwd_workspace_bytes_stored(int q_seq, int kv_len, int num_heads, int mode,
                                       int start_pos) {
    if (q_seq < 0 || kv_len < 0 || start_pos < 0 || num_heads < 1) return 0;
    if (mode != TA03_CAUSAL && mode != TA03_FULL && mode != TA03_CROSS) return 0;
    if (mode != TA03_CAUSAL && start_pos != 0) return 0;
    if (mode == TA03_CAUSAL && (long long)start_pos + q_seq > kv_len) return 0;
    if (mode == TA03_FULL && kv_len != q_seq) return 0;
    const ta03::DsLayout l{mode == TA03_CAUSAL ? 1 : 0, start_pos, q_seq, kv_len};
    const size_t tile_bytes = (size_t)ta03::kDsTile * ta03::kDsTile * sizeof(float);
    return attn_bwd_workspace_bytes(q_seq, num_heads) +
           (size_t)num_heads * (size_t)ta03::ds_tiles_per_head(l) * tile_bytes;
}

namespace {
// dS tiles per head that a backward workspace holds past the row-vector scratch.
long long bwd_tile_capacity(int q_seq, int num_heads, size_t workspace_bytes) {
    const size_t base = attn_bwd_workspace_bytes(q_seq, num_heads);
    const size_t tile_bytes = (size_t)ta03::kDsTile * ta03::kDsTile * sizeof(float);
    return workspace_bytes > base && q_seq > 0
        ? (long long)((workspace_bytes - base) / (tile_bytes * (size_t)num_heads)) : 0;
}
}  // namespace

int attn_bwd_windows(int q_seq, int kv_len, int num_heads, int mode, int start_pos,
                     size_t workspace_bytes) {
    if (attn_bwd_workspace_bytes_stored(q_seq, kv_len, num_heads, mode, start_pos) == 0 ||
        q_seq == 0)
        return 0;
    const ta03::DsLayout l{mode == TA03_CAUSAL ? 1 : 0, start_pos, q_seq, kv_len};
    return ta03::backward_windows(l, bwd_tile_capacity(q_seq, num_heads, workspace_bytes),
                                  ta03::kMaxBwdWindows);
}

int attn_bwd(const float* q, const float* k, const float* v, const float* out, const float* dout,
             const float* lse, float* dq, float* dk, float* dv, int q_seq, int kv_len,
             int num_heads, int num_kv_heads, int head_dim, int mode, int start_pos, float scale,
             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0) return TA03_ERR_SHAPE;
    if (q_seq < 0 || kv_len < 0 || start_pos < 0) return TA03_ERR_SHAPE;
    if (mode != TA03_CAUSAL && mode != TA03_FULL && mode != TA03_CROSS) return TA03_ERR_SHAPE;
    if (mode != TA03_CAUSAL && start_pos != 0) return TA03_ERR_SHAPE;
    if (mode == TA03_CAUSAL && (long long)start_pos + q_seq > kv_len) return TA03_ERR_SHAPE;
    if (mode == TA03_FULL && kv_len != q_seq) return TA03_ERR_SHAPE;
    if (!std::isfinite(scale)) return TA03_ERR_SHAPE;
    if (!head_dim_supported(head_dim)) return TA03_ERR_UNSUPPORTED;
    if ((long long)q_seq * num_heads * head_dim >= kMaxElems ||
        (long long)kv_len * num_kv_heads * head_dim >= kMaxElems)
        return TA03_ERR_UNSUPPORTED;
    // The kernels address 16 query rows or 32 key rows with 32-bit byte offsets.
    if ((long long)num_heads * head_dim >= (1ll << 24)) return TA03_ERR_UNSUPPORTED;
    if (q_seq == 0 && kv_len == 0) return TA03_OK;
    if (workspace_bytes < attn_bwd_workspace_bytes(q_seq, num_heads)) return TA03_ERR_WORKSPACE;
    if (q_seq > 0 && (q == nullptr || out == nullptr || dout == nullptr || lse == nullptr ||
                      dq == nullptr || workspace == nullptr))
        return TA03_ERR_NULL;
    if (kv_len > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
        return TA03_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
        !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
        !aligned16(workspace))
        return TA03_ERR_ALIGN;
    ta03::PrefillShape s;
    s.q_seq = q_seq;
    s.kv_len = kv_len;
    s.num_heads = num_heads;
    s.num_kv_heads = num_kv_heads;
    s.head_dim = head_dim;
    s.causal = mode == TA03_CAUSAL ? 1 : 0;
    s.start_pos = start_pos;
    s.scale = scale;
    s.q_stride = s.out_stride = (long long)num_heads * head_dim;
    s.k_stride = s.v_stride = (long long)num_kv_heads * head_dim;
    // Workspace past the row-vector scratch holds dS tiles (stored path): every tile
    // of the call, or a window of query tiles at a time.
    const size_t base = attn_bwd_workspace_bytes(q_seq, num_heads);
    const long long capacity = bwd_tile_capacity(q_seq, num_heads, workspace_bytes);
    float* ds = capacity > 0 ? static_cast<float*>(workspace) + base / sizeof(float) : nullptr;
    const hipError_t e = ta03::launch_backward(q, k, v, out, dout, lse, dq, dk, dv,
                                               static_cast<float*>(workspace), ds, capacity, s,
                                               stream);
    return e == hipSuccess ? TA03_OK : TA03_ERR_HIP;
}

int attn_rope_table(float* cos_sin, int rows, int head_dim, double theta, hipStream_t stream) {
    if (rows < 0 || head_dim < 2 || head_dim % 2 != 0) return TA03_ERR_SHAPE;
    if (!(theta > 0.0) || !std::isfinite(theta)) return TA03_ERR_SHAPE;
    if ((long long)rows * head_dim >= kMaxElems) return TA03_ERR_UNSUPPORTED;
    if (rows == 0) return TA03_OK;
    if (cos_sin == nullptr) return TA03_ERR_NULL;
    if (!aligned16(cos_sin)) return TA03_ERR_ALIGN;
    const hipError_t e = ta03::launch_rope_table(cos_sin, rows, head_dim, theta, stream);
    return e == hipSuccess ? TA03_OK : TA03_ERR_HIP;
}

int attn_fwd(const float* q, const float* k, const float* v, float* out, float* lse,
             int q_seq, int kv_len, int num_heads, int num_kv_heads, int head_dim,
             int mode, int start_pos, float scale, hipStream_t stream) {
    // Dense rows; full attention over the whole sequence.
    if (mode == TA03_FULL && kv_len != q_seq) return TA03_ERR_SHAPE;
    const long long qd = (long long)num_heads * head_dim;
    const long long kvd = (long long)num_kv_heads * head_dim;
    return attn_fwd_ex(q, qd, k, kvd, v, kvd, out, qd, lse, 0, q_seq, kv_len, num_heads,
                       num_kv_heads, head_dim, mode, start_pos, scale, stream);
}

size_t attn_decode_workspace_bytes(int num_heads, int num_kv_heads, int head_dim, int max_seq) {
    if (num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0 || max_seq < 1)
        return 0;
    if (!head_dim_supported(head_dim)) return 0;
    ta03::DecodeShape s{num_heads, num_kv_heads, head_dim, max_seq, 1.0f};
    return ta03::decode_plan(s, ta03::device_cu_count()).ws_floats * sizeof(float);
}

int attn_decode_workspace_init(void* workspace, size_t workspace_bytes, int num_heads,
                               int num_kv_heads, int head_dim, int max_seq, hipStream_t stream) {
    if (num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0 || max_seq < 1)
        return TA03_ERR_SHAPE;
    if (!head_dim_supported(head_dim)) return TA03_ERR_UNSUPPORTED;
    if (workspace == nullptr) return TA03_ERR_NULL;
    if (!aligned16(workspace)) return TA03_ERR_ALIGN;
    ta03::DecodeShape s{num_heads, num_kv_heads, head_dim, max_seq, 1.0f};
    const ta03::DecodePlan p = ta03::decode_plan(s, ta03::device_cu_count());
    if (workspace_bytes < p.ws_floats * sizeof(float)) return TA03_ERR_WORKSPACE;
    const hipError_t e = ta03::launch_decode_ws_init(static_cast<float*>(workspace), p, stream);
    return e == hipSuccess ? TA03_OK : TA03_ERR_HIP;
}

int attn_decode(const float* q, const float* k_cache, const float* v_cache,
                const uint32_t* kv_pos, float* out, float* lse,
                int num_heads, int num_kv_heads, int head_dim, int max_seq, float scale,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0 || max_seq < 1)
        return TA03_ERR_SHAPE;
    if (!std::isfinite(scale)) return TA03_ERR_SHAPE;
    if (!head_dim_supported(head_dim)) return TA03_ERR_UNSUPPORTED;
    if ((long long)max_seq * num_kv_heads * head_dim >= kMaxElems) return TA03_ERR_UNSUPPORTED;
    if (q == nullptr || k_cache == nullptr || v_cache == nullptr || kv_pos == nullptr ||
        out == nullptr || workspace == nullptr)
        return TA03_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        !aligned16(lse) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(kv_pos) & 3u) != 0)
        return TA03_ERR_ALIGN;
    ta03::DecodeShape s{num_heads, num_kv_heads, head_dim, max_seq, scale};
    const ta03::DecodePlan p = ta03::decode_plan(s, ta03::device_cu_count());
    if (workspace_bytes < p.ws_floats * sizeof(float)) return TA03_ERR_WORKSPACE;
    const hipError_t e = ta03::launch_decode(q, k_cache, v_cache, kv_pos, out, lse, s, p,
                                             static_cast<float*>(workspace), stream);
    return e == hipSuccess ? TA03_OK : TA03_ERR_HIP;
}

int attn_decode_noalloc(const float* q, const float* k_cache, const float* v_cache,
                        const uint32_t* kv_pos, float* out, float* lse, int num_heads,
                        int num_kv_heads, int head_dim, int max_seq, float scale,
                        hipStream_t stream) {
    if (num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0 || max_seq < 1)
        return TA03_ERR_SHAPE;
    if (!std::isfinite(scale)) return TA03_ERR_SHAPE;
    if (!head_dim_supported(head_dim)) return TA03_ERR_UNSUPPORTED;
    if ((long long)max_seq * num_kv_heads * head_dim >= kMaxElems) return TA03_ERR_UNSUPPORTED;
    if (q == nullptr || k_cache == nullptr || v_cache == nullptr || kv_pos == nullptr ||
        out == nullptr)
        return TA03_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        !aligned16(lse) || (reinterpret_cast<uintptr_t>(kv_pos) & 3u) != 0)
        return TA03_ERR_ALIGN;
    ta03::DecodeShape s{num_heads, num_kv_heads, head_dim, max_seq, scale};
    ta03::DecodePlan p = ta03::decode_plan(s, ta03::device_cu_count());
    // The scratch's own layout: the fixed counter region, then the partials.
    const size_t partials = p.ws_floats - p.part_offset;
    if (p.n_counters > ta03::kNoallocCounterWords ||
        partials > ta03::kNoallocScratchFloats - ta03::kNoallocCounterWords)
        return TA03_ERR_WORKSPACE;
    p.part_offset = ta03::kNoallocCounterWords;
    p.ws_floats = ta03::kNoallocCounterWords + partials;
    float* ws = nullptr;
    hipError_t e = ta03::noalloc_scratch(stream, &ws);
    if (e != hipSuccess) return TA03_ERR_HIP;
    e = ta03::launch_decode(q, k_cache, v_cache, kv_pos, out, lse, s, p, ws, stream);
    return e == hipSuccess ? TA03_OK : TA03_ERR_HIP;
}

int attn_decode_paged(const float* q, const float* k_pool, const float* v_pool, int num_pages,
                      int page_size, const int32_t* block_table, const uint32_t* kv_pos,
                      float* out, float* lse, int num_heads, int num_kv_heads, int head_dim,
                      int max_seq, float scale, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
    if (num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0 || max_seq < 1 ||
        num_pages < 1 || page_size < 1)
        return TA03_ERR_SHAPE;
    if (!std::isfinite(scale)) return TA03_ERR_SHAPE;
    if (!head_dim_supported(head_dim) || page_size % 16 != 0) return TA03_ERR_UNSUPPORTED;
    if ((long long)num_pages * page_size * num_kv_heads * head_dim >= (1ll << 40))
        return TA03_ERR_UNSUPPORTED;
    if (q == nullptr || k_pool == nullptr || v_pool == nullptr || block_table == nullptr ||
        kv_pos == nullptr || out == nullptr || workspace == nullptr)
        return TA03_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
        !aligned16(lse) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(kv_pos) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0)
        return TA03_ERR_ALIGN;
    ta03::DecodeShape s{num_heads, num_kv_heads, head_dim, max_seq, scale};
    const ta03::DecodePlan p = ta03::decode_plan(s, ta03::device_cu_count());
    if (workspace_bytes < p.ws_floats * sizeof(float)) return TA03_ERR_WORKSPACE;
    if (ta03::decode_table_lds_bytes(s, p, page_size) > 64 * 1024) return TA03_ERR_UNSUPPORTED;
    const hipError_t e = ta03::launch_decode(q, k_pool, v_pool, kv_pos, out, lse, s, p,
                                             static_cast<float*>(workspace), stream,
                                             block_table, page_size, num_pages);
    return e == hipSuccess ? TA03_OK : TA03_ERR_HIP;
}

int attn_set_kernel_override(int knob, int value) {
    switch (knob) {
        case TA03_OVERRIDE_PREFILL_ROWS:
            if (value != 0 && value != 16 && value != 32) return TA03_ERR_SHAPE;
            ta03::g_prefill_rows.store(value, std::memory_order_relaxed);
            return TA03_OK;
        case TA03_OVERRIDE_BWD_PATH:
            if (value < 0 || value > 2) return TA03_ERR_SHAPE;
            ta03::g_bwd_path.store(value, std::memory_order_relaxed);
            return TA03_OK;
        default:
            return TA03_ERR_SHAPE;
    }
}

const char* attn_strerror(int status) {
    switch (status) {
        case TA03_OK: return "ok";
        case TA03_ERR_NULL: return "a required pointer is NULL";
        case TA03_ERR_SHAPE: return "inconsistent or invalid sizes";
        case TA03_ERR_UNSUPPORTED: return "unsupported head_dim or size";
        case TA03_ERR_WORKSPACE: return "decode workspace too small";
        case TA03_ERR_HIP: return "HIP kernel launch failed";
        case TA03_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        default: return "unknown status";
    }
}

}  // extern "C"
