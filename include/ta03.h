/*
 * ta03.h -- C ABI of the MI355X (gfx950) fused attention forward.
 *
 *   out = softmax(scale * Q * K^T + mask) * V      (one pass, online softmax)
 *
 * with the per-(row, head) side output (max score, log of the sum of
 * exp(score - max)). The operation and its conventions are those of three
 * WGSL shaders:
 *   - meganeura "attention.wgsl": whole-sequence tiled attention. Header
 *     comment: the causal (window pos+1), full (window q_seq) and cross
 *     (window kv_seq) variants. main(): GQA map kv_head = head /
 *     (num_heads / num_kv_heads); running max starts at -1e30; the result is
 *     divided by a zero-safe sum; the side output stores (max, log(sum)) and
 *     -1e30 for log(0) "for the backward pass".
 *   - meganeura "cached_attention.wgsl": one query token over a KV cache; the
 *     cache position kv_pos is read from a device buffer and the window is
 *     [0, kv_pos].
 *   - cera "attention_prefill.wgsl": a batch of queries continuing a cache
 *     from start_pos; query i attends to [0, start_pos + i]; header
 *     "Constraints": head_dim <= 128 and the cache must hold start_pos +
 *     n_queries valid rows, with a defensive clamp of the window to the cache.
 *
 * Layouts (all f32, dense, row-major, device memory):
 *   q, out : [q_seq, num_heads * head_dim]       head h at columns h*head_dim
 *   k, v   : [rows,  num_kv_heads * head_dim]    rows >= the window's end
 *   lse    : [q_seq, num_heads, 2]               (max, log sum exp(s - max))
 * Every tensor pointer must be 16-byte aligned.
 *
 * Ownership: the caller owns every buffer, the workspace and the stream. The
 * library allocates nothing, frees nothing and never synchronises: each call
 * validates its arguments on the host, enqueues its kernels on `stream` and
 * returns. Invalid arguments are rejected before any HIP call is made, so
 * nothing is enqueued on an error return.
 *
 * Thread safety: calls are independent; two calls that write the same
 * buffers (or share one decode workspace) must be ordered by the caller.
 */
#ifndef TA03_H
#define TA03_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Masking variant (meganeura attention.wgsl, header comment). */
typedef enum {
    TA03_CAUSAL = 0, /* row i sees keys [0, min(start_pos + i + 1, kv_len)) */
    TA03_FULL = 1,   /* every row sees [0, kv_len); requires kv_len == q_seq */
    TA03_CROSS = 2   /* every row sees [0, kv_len); any kv_len >= 0 */
} ta03_mode;

typedef enum {
    TA03_OK = 0,
    TA03_ERR_NULL = -1,        /* a required pointer is NULL */
    TA03_ERR_SHAPE = -2,       /* inconsistent sizes (see each entry point) */
    TA03_ERR_UNSUPPORTED = -3, /* head_dim outside {64, 128}, or a size too large */
    TA03_ERR_WORKSPACE = -4,   /* decode workspace smaller than required */
    TA03_ERR_HIP = -5,         /* a kernel launch failed (hipGetLastError) */
    TA03_ERR_ALIGN = -6        /* a pointer is not 16-byte aligned */
} ta03_status;

/*
 * attn_fwd -- prefill: whole-sequence causal / full / cross attention
 * (meganeura attention.wgsl, main) and batched causal prefill continuing a
 * cache from start_pos (cera attention_prefill.wgsl, main).
 *
 *   q        [q_seq, num_heads*head_dim]
 *   k, v     [>= kv_len, num_kv_heads*head_dim]; only rows [0, kv_len) that
 *            some row's window covers are read (may be NULL if kv_len == 0)
 *   out      [q_seq, num_heads*head_dim], written in full
 *   lse      [q_seq, num_heads, 2] or NULL; lse[i,h] = (m, log Z) with
 *            m = max_j s_ij and Z = sum_j exp(s_ij - m), both natural-log
 *            units; an empty window writes out = 0 and lse = (-1e30, -1e30)
 *   mode     ta03_mode
 *   start_pos causal offset of row 0 (0 unless mode == TA03_CAUSAL)
 *   scale    multiplies Q.K^T (the pages use 1/sqrt(head_dim))
 *
 * Errors: TA03_ERR_NULL for a NULL q/out (or k/v with kv_len > 0);
 * TA03_ERR_SHAPE if num_heads, num_kv_heads < 1, num_heads % num_kv_heads,
 * q_seq, kv_len or start_pos < 0, mode unknown, start_pos != 0 outside
 * causal mode, causal start_pos + q_seq > kv_len (the pages' host assert), a
 * full call with kv_len != q_seq, or a non-finite scale;
 * TA03_ERR_UNSUPPORTED for head_dim not in {64, 128}; TA03_ERR_ALIGN;
 * TA03_ERR_HIP. q_seq == 0 is a valid no-op. Same as attn_fwd_ex with dense
 * row strides and q_base = 0.
 */
int attn_fwd(const float* q, const float* k, const float* v, float* out, float* lse,
             int q_seq, int kv_len, int num_heads, int num_kv_heads, int head_dim,
             int mode, int start_pos, float scale, hipStream_t stream);

/*
 * attn_fwd_ex -- attn_fwd over strided rows and a sub-batch of the query
 * batch: the parameter block of cera attention_prefill.wgsl (header and
 * main: q_stride, out_stride, q_base; q_global = q_base + i addresses the
 * rows and sets the causal position start_pos + q_global).
 *
 *   q_stride, out_stride  floats between consecutive rows of q / out
 *                         (>= num_heads*head_dim), e.g. the row length of a
 *                         fused QKV buffer
 *   k_stride, v_stride    floats between consecutive cache rows
 *                         (>= num_kv_heads*head_dim)
 *   q_base                first row of q / out (and lse) this call handles;
 *                         rows [q_base, q_base + q_seq) are read and written
 *   lse                   [q_base + q_seq, num_heads, 2] rows, indexed by the
 *                         global row, or NULL
 *
 * Causal rows see [0, min(start_pos + q_base + i + 1, kv_len)); full and
 * cross rows see [0, kv_len) (full: q_base + q_seq <= kv_len). Strides must be
 * multiples of 4 floats (TA03_ERR_ALIGN) and below 2^31
 * (TA03_ERR_UNSUPPORTED). Otherwise as attn_fwd: TA03_ERR_SHAPE also for
 * q_base < 0, a stride shorter than a row, or causal start_pos + q_base +
 * q_seq > kv_len.
 */
int attn_fwd_ex(const float* q, long long q_stride, const float* k, long long k_stride,
                const float* v, long long v_stride, float* out, long long out_stride,
                float* lse, int q_base, int q_seq, int kv_len, int num_heads,
                int num_kv_heads, int head_dim, int mode, int start_pos, float scale,
                hipStream_t stream);

/*
 * attn_fwd_rope -- attn_fwd_ex with a rotary position embedding applied to
 * the queries and keys as the kernel loads them. meganeura attention.wgsl
 * (main) routes each loaded query element through a rotation hook and builds
 * each key element through a hook expression, but the page gives no formula;
 * the rotation read into those hooks is the rotate-half form: in every head,
 * element e < head_dim/2 pairs with element e + head_dim/2 and, at position p,
 *     x'[e]       = x[e] * cos - x[e + head_dim/2] * sin
 *     x'[e + d/2] = x[e + d/2] * cos + x[e] * sin
 * with (cos, sin) = rope_cs[p][e]. The query of global row q_base + i sits at
 * position start_pos + q_base + i (start_pos is 0 outside causal mode), key
 * row j at position j. q and k are not modified.
 *
 *   rope_cs    device, [rope_rows, head_dim/2, 2] floats, 16-byte aligned:
 *              the (cos, sin) pair of every (position, pair); attn_rope_table
 *              fills the standard table, any other table is used as given
 *   rope_rows  rows of rope_cs; must cover every position used:
 *              >= max(start_pos + q_base + q_seq, kv_len)
 *
 * Errors as attn_fwd_ex, plus TA03_ERR_NULL for a NULL rope_cs,
 * TA03_ERR_ALIGN for a misaligned one, TA03_ERR_SHAPE for too few rope_rows
 * (q_seq > 0), TA03_ERR_UNSUPPORTED for rope_rows * head_dim >= 2^31.
 */
int attn_fwd_rope(const float* q, long long q_stride, const float* k, long long k_stride,
                  const float* v, long long v_stride, float* out, long long out_stride,
                  float* lse, int q_base, int q_seq, int kv_len, int num_heads,
                  int num_kv_heads, int head_dim, int mode, int start_pos, float scale,
                  const float* rope_cs, int rope_rows, hipStream_t stream);

/*
 * attn_fwd_rope_q -- attn_fwd_rope for keys that are already turned (a cache
 * that stores rotated keys, or keys passed once through attn_rope_apply): the
 * queries are turned as the kernel loads them, exactly as in attn_fwd_rope,
 * and k is used as given. The same rotation read into the pages' hooks
 * (meganeura attention.wgsl, main), split so that each key is turned once
 * per call instead of once per block of query rows that reads it. Arguments,
 * layouts and errors as attn_fwd_rope, except that rope_rows must cover the
 * query positions only: >= start_pos + q_base + q_seq.
 */
int attn_fwd_rope_q(const float* q, long long q_stride, const float* k, long long k_stride,
                    const float* v, long long v_stride, float* out, long long out_stride,
                    float* lse, int q_base, int q_seq, int kv_len, int num_heads,
                    int num_kv_heads, int head_dim, int mode, int start_pos, float scale,
                    const float* rope_cs, int rope_rows, hipStream_t stream);

/*
 * attn_rope_apply -- turn rows by the rotary table, the rotation
 * attn_fwd_rope applies to keys as it loads them: for row r < rows, head
 * h < heads and pair e < head_dim/2, at position pos0 + r with
 * (cos, sin) = rope_cs[pos0 + r][e],
 *     y[r][h*head_dim + e]              = x[..e] * cos - x[..e + head_dim/2] * sin
 *     y[r][h*head_dim + e + head_dim/2] = x[..e + head_dim/2] * cos + x[..e] * sin
 * Columns past heads * head_dim are not touched.
 *
 *   x, y      device, rows x heads * head_dim floats with row strides
 *             x_stride, y_stride (floats, multiples of 4), 16-byte aligned;
 *             y == x with y_stride == x_stride turns in place, any other
 *             overlap is rejected
 *   rope_cs   device, [rope_rows, head_dim/2, 2] floats, 16-byte aligned
 *             (attn_rope_table), rope_rows >= pos0 + rows
 *
 * Errors: TA03_ERR_SHAPE for rows < 0, heads < 1, pos0 < 0, head_dim not a
 * positive multiple of 8, a stride below heads * head_dim, too few rope_rows
 * or overlapping x and y; TA03_ERR_UNSUPPORTED for a stride, heads *
 * head_dim or rope_rows * head_dim >= 2^31; TA03_ERR_NULL; TA03_ERR_ALIGN;
 * TA03_ERR_HIP. rows == 0 is a no-op.
 */
int attn_rope_apply(const float* x, long long x_stride, float* y, long long y_stride, int rows,
                    int heads, int head_dim, int pos0, const float* rope_cs, int rope_rows,
                    hipStream_t stream);

/*
 * attn_rope_table -- fill the standard rotary table for attn_fwd_rope:
 * cos_sin[p][e] = (cos(a), sin(a)), a = p * theta^(-2e/head_dim), for
 * p < rows and e < head_dim/2 (the frequencies of the common rotary
 * embedding; the pages name no base, theta is the caller's, e.g. 10000).
 * Each angle and its cosine and sine are computed in double precision and
 * rounded once to float.
 *
 *   cos_sin   device, rows * head_dim floats, 16-byte aligned, written in full
 *
 * Errors: TA03_ERR_SHAPE for rows < 0, head_dim < 2 or odd, theta not
 * finite and positive; TA03_ERR_UNSUPPORTED for rows * head_dim >= 2^31;
 * TA03_ERR_NULL; TA03_ERR_ALIGN; TA03_ERR_HIP. rows == 0 is a no-op.
 */
int attn_rope_table(float* cos_sin, int rows, int head_dim, double theta, hipStream_t stream);

/*
 * attn_bwd -- gradients of attn_fwd (dense rows, no rotation) for a loss
 * whose gradient with respect to out is dout. meganeura attention.wgsl keeps
 * the pair lse = (m, log l) "for backward" without giving one; this is the
 * exact derivative of the forward's definition, built on that pair:
 *   P_ij = exp(s_ij - m_i - log l_i),  s_ij = scale <q_i, k_j>, j in row i's window
 *   D_i = <dout_i, out_i>,  dS_ij = P_ij (<dout_i, v_j> - D_i)
 *   dq_i = scale sum_j dS_ij k_j
 *   dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dout_i
 * with dk and dv summed over the query heads of each KV head.
 *
 *   q, out, dout  [q_seq, num_heads*head_dim]: the forward's inputs and
 *                 output, and the loss gradient
 *   k, v          [>= kv_len, num_kv_heads*head_dim]; rows [0, kv_len) read
 *   lse           [q_seq, num_heads, 2] as the forward with these inputs
 *                 wrote it (required)
 *   dq            [q_seq, num_heads*head_dim], written in full
 *   dk, dv        [kv_len, num_kv_heads*head_dim], written in full (0 for
 *                 keys no row sees)
 *   mode, start_pos, scale  as the forward
 *   workspace     device scratch, 16-byte aligned, overwritten: at least
 *                 attn_bwd_workspace_bytes(q_seq, num_heads) bytes (two
 *                 floats per row and head: D_i and the row's exponent offset).
 *                 The bytes past that hold score gradients dS_ij in 16 x 16
 *                 tiles (1 KiB per tile and head), which lets dq be formed
 *                 from them instead of recomputing the scores:
 *                 attn_bwd_workspace_bytes_stored(q_seq, kv_len, num_heads,
 *                 mode, start_pos) bytes hold every tile of the call (4 bytes
 *                 per (row, key) pair in the windows, per head, rounded up to
 *                 whole tiles); any smaller workspace that holds the tiles of
 *                 the call's longest 16-row query tile runs the stored path in
 *                 windows of whole query tiles (attn_bwd_windows)
 *
 * Stored path: D_i, then per window of query tiles the dk/dv kernel over the
 * window's rows, storing its dS tiles (dk, dv written by the first window,
 * added to by the later ones), and dq of the window's rows from the tiles
 * (three launches when every tile fits). With n windows, window w holds the
 * query tiles w, w + n, w + 2n, ... (every window spans the whole sequence). Recompute path: two launches (dq
 * with D_i, recomputing the scores; dk, dv). The stored path is taken when
 * the call is long enough for it to pay (the dq grid over the tiles fills the
 * device's compute units) and the workspace needs at most 32 windows;
 * otherwise the call recomputes.
 * attn_set_kernel_override can force either path (testing). Both
 * paths run on stream with no allocation and no atomics (results are
 * run-to-run identical; the two paths agree to rounding). Errors: as attn_fwd for the sizes and mode;
 * TA03_ERR_NULL for a NULL q, out, dout, lse, dq or workspace (q_seq > 0) or
 * k, v, dk, dv (kv_len > 0); TA03_ERR_WORKSPACE for a short workspace;
 * TA03_ERR_UNSUPPORTED for q_seq*num_heads*head_dim or
 * kv_len*num_kv_heads*head_dim >= 2^31, or num_heads*head_dim >= 2^24;
 * TA03_ERR_ALIGN; TA03_ERR_HIP.
 * q_seq == 0 and kv_len == 0 is a no-op; q_seq == 0 alone writes zero dk, dv.
 */
size_t attn_bwd_workspace_bytes(int q_seq, int num_heads);
/* Workspace bytes for the stored path: attn_bwd_workspace_bytes(q_seq,
 * num_heads) + num_heads * T * 1024, T the 16 x 16 tiles of one head's
 * windows; 0 for sizes attn_bwd rejects. */
size_t attn_bwd_workspace_bytes_stored(int q_seq, int kv_len, int num_heads, int mode,
                                       int start_pos);

/*
 * attn_bwd_windows -- host-only query: the number of windows of query tiles
 * in which attn_bwd's stored path runs with a workspace of workspace_bytes
 * for these sizes (the fewest n for which every window w < n, the 16-row
 * query tiles w, w + n, w + 2n, ..., holds at most the dS tiles that fit past
 * the row-vector scratch). 1 when every tile fits. 0 when no count up to 32 fits
 * (the workspace is below the tiles of the longest query tile, or more than
 * 32 windows would be needed), for q_seq == 0 and for invalid sizes (as
 * attn_bwd_workspace_bytes_stored); attn_bwd then recomputes. Whether a call
 * with a count above 0 takes the stored path also depends on its size (see
 * attn_bwd). Touches no device.
 */
int attn_bwd_windows(int q_seq, int kv_len, int num_heads, int mode, int start_pos,
                     size_t workspace_bytes);
int attn_bwd(const float* q, const float* k, const float* v, const float* out, const float* dout,
             const float* lse, float* dq, float* dk, float* dv, int q_seq, int kv_len,
             int num_heads, int num_kv_heads, int head_dim, int mode, int start_pos, float scale,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode_workspace_bytes -- bytes of device workspace attn_decode needs
 * for these sizes: split-KV partial results (per query head and split, an
 * unnormalised output row plus its max and sum) and one completion counter
 * per (kv head, head block). Returns 0 for invalid sizes.
 */
size_t attn_decode_workspace_bytes(int num_heads, int num_kv_heads, int head_dim,
                                   int max_seq);

/*
 * attn_decode_workspace_init -- enqueue on `stream` the zero fill of the
 * completion counters of a decode workspace (one small kernel; no memset
 * node, so it may also be captured in a graph). Same size arguments as
 * attn_decode_workspace_bytes. Errors: TA03_ERR_SHAPE, TA03_ERR_UNSUPPORTED,
 * TA03_ERR_NULL, TA03_ERR_ALIGN, TA03_ERR_WORKSPACE, TA03_ERR_HIP.
 */
int attn_decode_workspace_init(void* workspace, size_t workspace_bytes, int num_heads,
                               int num_kv_heads, int head_dim, int max_seq,
                               hipStream_t stream);

/*
 * attn_decode -- one query token over a KV cache (meganeura
 * cached_attention.wgsl, main). The window is [0, min(*kv_pos + 1,
 * max_seq)): kv_pos lives in device memory (a uint32 written by earlier
 * device work), so a captured launch can be replayed as the cache grows;
 * the clamp to max_seq is the defensive clamp of cera
 * attention_prefill.wgsl. Equivalent to attn_fwd(TA03_CAUSAL, q_seq = 1,
 * start_pos = window - 1, kv_len = window).
 *
 *   q          [1, num_heads*head_dim]
 *   k_cache,
 *   v_cache    [max_seq, num_kv_heads*head_dim]
 *   kv_pos     device pointer to one uint32 (4-byte aligned)
 *   out        [1, num_heads*head_dim]
 *   lse        [1, num_heads, 2] or NULL (same convention as attn_fwd)
 *   workspace  device scratch of at least attn_decode_workspace_bytes(...)
 *              bytes, owned by the caller. It holds the split partials and
 *              one completion counter per (kv head, head block); it must be
 *              zero-filled before its first use (attn_decode_workspace_init,
 *              or any zero fill). Every call leaves the counters at zero, so
 *              a workspace is reused, or a captured call replayed, without
 *              re-initialisation. Calls sharing a workspace must be ordered
 *              on one stream.
 *
 * Errors: TA03_ERR_NULL, TA03_ERR_SHAPE (num_heads, num_kv_heads, max_seq
 * < 1, num_heads % num_kv_heads, non-finite scale), TA03_ERR_UNSUPPORTED,
 * TA03_ERR_WORKSPACE, TA03_ERR_ALIGN, TA03_ERR_HIP.
 */
int attn_decode(const float* q, const float* k_cache, const float* v_cache,
                const uint32_t* kv_pos, float* out, float* lse,
                int num_heads, int num_kv_heads, int head_dim, int max_seq, float scale,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): same arguments, results and
 * errors as attn_decode, bit for bit, without the workspace. The split
 * partials and completion counters live in a fixed 4 MiB device array inside
 * the library, one per GPU, held until the process ends; the call allocates
 * nothing and frees nothing. Its first call on a device looks up that
 * array's address and enqueues the zero fill of its counters on `stream`;
 * every call leaves the counters at zero.
 *
 * Limits: at most 256 (kv head, head block) groups, i.e. num_kv_heads *
 * ceil(group / 4) <= 256, and num_heads * n_splits * (head_dim + 4) floats of
 * partials <= 1032192, n_splits being about the device's compute units per
 * group (on a 256-CU device at most 135168 floats for any head count);
 * larger shapes return TA03_ERR_WORKSPACE before any HIP call.
 *
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or threads) race and must be ordered by the
 * caller, as calls that share an attn_decode workspace must.
 */
int attn_decode_noalloc(const float* q, const float* k_cache, const float* v_cache,
                        const uint32_t* kv_pos, float* out, float* lse, int num_heads,
                        int num_kv_heads, int head_dim, int max_seq, float scale,
                        hipStream_t stream);

/*
 * attn_decode_paged -- attn_decode over a paged KV cache. The pages call
 * caches too long for one binding "future paged-KV work" (cera
 * attention_prefill.wgsl, header) without giving a layout; this one is:
 *
 *   k_pool, v_pool  [num_pages, page_size, num_kv_heads*head_dim]: page p
 *                   holds page_size consecutive token rows in the dense
 *                   cache's row layout
 *   block_table     device int32 [ceil(max_seq / page_size)]: token t lives
 *                   in row t % page_size of page block_table[t / page_size];
 *                   entries outside [0, num_pages) are clamped on the device
 *                   (never an out-of-bounds read; the result is then
 *                   meaningless)
 *   page_size       a multiple of 16 tokens
 *   max_seq         token capacity covered by the table
 *
 * kv_pos, window, q, out, lse and the workspace (same size and rules as
 * attn_decode for the same num_heads, num_kv_heads, head_dim, max_seq) are
 * as in attn_decode. Errors as attn_decode, plus TA03_ERR_SHAPE for
 * num_pages or page_size < 1, TA03_ERR_UNSUPPORTED for a page_size that is
 * not a multiple of 16 or a table slice too large for one block's LDS.
 */
int attn_decode_paged(const float* q, const float* k_pool, const float* v_pool, int num_pages,
                      int page_size, const int32_t* block_table, const uint32_t* kv_pos,
                      float* out, float* lse, int num_heads, int num_kv_heads, int head_dim,
                      int max_seq, float scale, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * attn_set_kernel_override -- testing hook: force one kernel choice for every
 * later call in this process (all threads), so that a shape can be run
 * through each kernel that can serve it. value 0 restores the automatic
 * choice, which every other caller should keep. Results of any choice match
 * the definition to the stated tolerances; only speed differs.
 *
 *   TA03_OVERRIDE_PREFILL_ROWS  16 or 32: the 16-row or the 32-row prefill
 *                               kernel for calls without rotation
 *   TA03_OVERRIDE_BWD_PATH      1: attn_bwd takes the stored-dS path whenever
 *                               its workspace holds every tile; 2: the
 *                               recompute path
 *
 * Errors: TA03_ERR_SHAPE for an unknown knob or value. No HIP call is made.
 */
enum { TA03_OVERRIDE_PREFILL_ROWS = 1, TA03_OVERRIDE_BWD_PATH = 2 };
int attn_set_kernel_override(int knob, int value);

/* attn_strerror -- static description of a ta03_status value. */
const char* attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* TA03_H */
