/*
 * diffkv_attn.h - paged attention for models whose key and value head dims
 * differ (QK 192, V 128), with grouped-query heads, on MI355X (gfx950).
 *
 * What the calls compute (the pages this library is built from):
 *   - "sglang PR 41886, Default MiMo attention to FA4 on SM100", Accuracy
 *     Tests: QK=192/V=128 attention, full and sliding-window layers with
 *     sinks, single-token decode, 8-token verify, ragged page boundaries,
 *     graph replay.
 *   - "diffbot/MiMo-V2.6-Flash-RL-FP8KV-W4A8-2x-RTX-PRO-6000", What the
 *     kernels do: split-KV for the multi-token verify step, 4096-token
 *     prefill chunks at 26K context with 16 query heads per KV head, FP8
 *     E4M3 K/V converted as it is loaded.
 *   - "sglang PR 32818, Route asymmetric-KV models to fa4 on SM100": K and V
 *     rows have different widths, so they live in two separate caches; a
 *     model's layer types may carry their own head-dim pairs (the change's
 *     asymmetric-KV property), so the QK width D_qk is 192 or, for
 *     symmetric heads, 128 (V stays 128).
 *
 * For sequence b with L = seq_lens[b] and n = q_lens[b], new token i (packed
 * row r0 + i, r0 = q_lens[0] + ... + q_lens[b-1]) sits at position
 * p = L - n + i and, for query head h, attends over KV head g = h / G
 * (G = num_q_heads / num_kv_heads) to the keys j with lo <= j <= p, where
 * lo = 0 when window <= 0 and lo = max(0, p - window + 1) otherwise:
 *     x_j  = softmax_scale * dot(q[r0+i, h, :], K_j)
 *     out  = sum_j e^(x_j - m) V_j / (sum_j e^(x_j - m) + e^(s_h - m))
 * with K_j = k_cache[block_table[b][j / P], j % P, g, :] * k_scale,
 * V_j likewise with v_scale (scales apply to FP8 caches only; bf16 caches are
 * used as stored), m the running maximum, and the sink term present only
 * when sinks != NULL.  s_h is a logit in the already-scaled domain.
 *
 * All four entry points compute this same function; they differ only in
 * how the work is cut up and in the q_len they accept.
 */
#ifndef DIFFKV_ATTN_H
#define DIFFKV_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  No exception ever crosses this interface. */
enum {
  DIFFKV_OK = 0,
  DIFFKV_INVALID_ARGUMENT = 1,   /* null required pointer, bad size or bound   */
  DIFFKV_UNSUPPORTED = 2,        /* head dims, page size or dtype not built     */
  DIFFKV_WORKSPACE_TOO_SMALL = 3,/* workspace_bytes below diffkv_attn_workspace_bytes */
  DIFFKV_HIP_ERROR = 4           /* a launch failed (hipGetLastError)           */
};

/* Entry selectors for diffkv_attn_workspace_bytes / diffkv_attn_validate. */
enum { DIFFKV_ENTRY_DECODE = 0, DIFFKV_ENTRY_VERIFY = 1, DIFFKV_ENTRY_PREFILL = 2,
       DIFFKV_ENTRY_MIXED = 3 };

/* K/V storage formats. */
enum {
  DIFFKV_KV_BF16 = 0,            /* bfloat16                                    */
  DIFFKV_KV_FP8_E4M3 = 1         /* OCP FP8 E4M3FN (bias 7, max 448, NaN 0x7F/0xFF) */
};

/*
 * Shape descriptor.  Every field is a host-side value; the launch grid is
 * derived from these bounds only, never from device data, so a call can be
 * captured in a HIP graph and replayed with new device contents of seq_lens,
 * q_lens and block_table as long as they stay within these bounds.
 */
typedef struct diffkv_attn_desc {
  int32_t batch;               /* number of sequences B >= 1                        */
  int32_t num_q_heads;         /* Hq >= 1                                           */
  int32_t num_kv_heads;        /* Hkv >= 1, Hq % Hkv == 0, G = Hq / Hkv             */
  int32_t head_dim_qk;         /* D_qk: 192, or 128 for symmetric 128/128 heads     */
  int32_t head_dim_v;          /* must be 128                                       */
  int32_t page_size;           /* P: a power of two in [1, 256]                     */
  int32_t num_pages;           /* pages in each cache                               */
  int32_t block_table_stride;  /* int32 entries per block-table row                 */
  int32_t max_seq_len;         /* >= every seq_lens[b]                              */
  int32_t max_q_len;           /* >= every q_lens[b]; 1 for decode, <= 16 for verify */
  int32_t total_q;             /* == sum of q_lens: rows of q and out               */
  int32_t kv_dtype;            /* DIFFKV_KV_BF16 or DIFFKV_KV_FP8_E4M3              */
  int32_t force_num_splits;    /* 0 = automatic; 1..65536 forces the key-axis split
                                  count (decode, verify and mixed's split-KV part; a
                                  test hook)                                        */
  /* Measurement hook: two caller-created HIP events, or both NULL.  When
   * set, the call dispatches its first main kernel (not the split merge;
   * for mixed, the split-KV kernel) with them as start and stop events
   * (hipExtLaunchKernel), so hipEventElapsedTime(start, stop) is that
   * kernel's execution time.  A call that fails before its launch leaves
   * them as they were.  Exactly one NULL is DIFFKV_INVALID_ARGUMENT.       */
  hipEvent_t profile_start;
  hipEvent_t profile_stop;
} diffkv_attn_desc;

/*
 * Attention over the paged cache.  Layouts (all row-major, contiguous):
 *   q            bf16  [total_q, Hq, D_qk]; sequence b's rows start at r0
 *   k_cache      bf16 or E4M3 [num_pages, P, Hkv, D_qk]
 *   v_cache      bf16 or E4M3 [num_pages, P, Hkv, 128]
 *   block_table  int32 [batch, block_table_stride]; entry t is the physical
 *                page of the sequence's tokens [t*P, (t+1)*P).  Only entries
 *                of pages holding a visible key are read; the others (pages
 *                past the end, pages wholly before the window) may hold any
 *                value, e.g. -1.
 *   seq_lens     int32 [batch], tokens in the cache including the new ones
 *   q_lens       int32 [batch], new tokens per sequence; NULL means all 1
 *   window       keys visible to a token: the `window` newest up to and
 *                including itself; <= 0 means full attention
 *   sinks        fp32 [Hq] per-query-head sink logits, or NULL
 *   k_scale, v_scale  per-tensor dequantisation scales (FP8 caches only)
 *   softmax_scale     multiplies q.k before the softmax
 *   out          bf16  [total_q, Hq, 128], written (round to nearest even)
 *   lse_out      fp32  [total_q, Hq] natural-log log-sum-exp of the key
 *                logits (sink excluded), or NULL; the row sums behind it
 *                add the bf16-rounded probabilities the P.V product uses,
 *                so it is exact to about 2^-8
 *   count_out    int32 [total_q, Hq]: number of keys each row combined, or
 *                NULL (a check on which slots are read; costs time)
 *   workspace    device scratch of at least diffkv_attn_workspace_bytes(desc,
 *                entry) bytes, or NULL when that is 0; clobbered
 *   stream       HIP stream every kernel is enqueued on, in order
 *
 * Ownership: every pointer is caller-owned device memory; the library keeps
 * no reference after returning, never allocates, frees or synchronises, and
 * never reads device data on the host.  out must not alias an input.
 *
 * Thread safety: every call is re-entrant.  The library's only state is the
 * compute-unit count of each device (filled once per device under
 * std::call_once), and the device address of the allocation-free verify
 * entry's static workspace (also once per device).
 *
 * Preconditions on device data (undefined behaviour if broken; the debug
 * build checks them, see diffkv_attn_debug_flags):
 *   1 <= q_lens[b] <= seq_lens[b] <= max_seq_len, q_lens[b] <= max_q_len,
 *   sum(q_lens) == total_q, and every block-table entry that is read lies in
 *   [0, num_pages).  Slots the rows cannot see may hold anything, NaN
 *   included; it never reaches the output.
 *
 * Returns DIFFKV_OK, or a status from the enum above (synchronous checks of
 * the descriptor and pointers, or a launch failure).  Faults in device code
 * surface as HIP errors at the caller's next synchronisation.
 *
 * diffkv_attn_decode:  max_q_len must be 1 (single-token decode, split-KV).
 * diffkv_attn_verify:  max_q_len <= 16 (speculative verify block, causal
 *                      within the block, split-KV so long contexts fill the
 *                      GPU, as the split-KV fix for the verify step does).
 * diffkv_attn_prefill: any q_len (chunked causal prefill over a paged prefix,
 *                      large query tiles on the matrix cores).
 * diffkv_attn_mixed:   any q_len per sequence, for batches that mix decode,
 *                      verify and prefill sequences ("sammysun0711/sglang PR
 *                      35", file table: ordinary decode prepared alongside
 *                      speculative verify; "diffbot/MiMo-V2.6-Flash-RL-FP8KV-
 *                      W4A8-2x-RTX-PRO-6000", Credits: mixed-batch changes):
 *                      the sequences with q_len <= 16 take the split-KV kernels,
 *                      the others the prefill kernel, both enqueued on
 *                      `stream` in that order.  Which path a sequence takes
 *                      is decided on the device from q_lens, so the launch
 *                      shapes still depend on the descriptor alone.
 */
int diffkv_attn_decode(const diffkv_attn_desc* desc, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* q_lens, int32_t window, const float* sinks, float k_scale,
                       float v_scale, float softmax_scale, void* out, float* lse_out,
                       int32_t* count_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

int diffkv_attn_verify(const diffkv_attn_desc* desc, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* q_lens, int32_t window, const float* sinks, float k_scale,
                       float v_scale, float softmax_scale, void* out, float* lse_out,
                       int32_t* count_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

int diffkv_attn_prefill(const diffkv_attn_desc* desc, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                        const int32_t* q_lens, int32_t window, const float* sinks, float k_scale,
                        float v_scale, float softmax_scale, void* out, float* lse_out,
                        int32_t* count_out, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

int diffkv_attn_mixed(const diffkv_attn_desc* desc, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* q_lens, int32_t window, const float* sinks, float k_scale,
                      float v_scale, float softmax_scale, void* out, float* lse_out,
                      int32_t* count_out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * diffkv_attn_verify without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, layouts, results and errors
 * are those of diffkv_attn_verify (bitwise the same output); the split-KV
 * partials go to a static 32 MiB array the library holds on each device it
 * runs on (zero-filled when the library loads, kept until the process ends).
 * The call allocates and frees nothing.  A call whose split needs more than
 * 32 MiB of workspace (264 bytes per partial row, so about 127K rows; the
 * long-verify shape, 4 blocks of 8 tokens at GQA 8, needs 4.4 MB) returns
 * DIFFKV_WORKSPACE_TOO_SMALL without launching.
 * Every call on one device shares that device's array, which keeps the last
 * call's contents: calls that overlap on one device (two streams, or two
 * host threads) race and must be serialised by the caller.
 */
int diffkv_attn_verify_noalloc(const diffkv_attn_desc* desc, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* q_lens, int32_t window,
                               const float* sinks, float k_scale, float v_scale,
                               float softmax_scale, void* out, float* lse_out, int32_t* count_out,
                               hipStream_t stream);

/*
 * Context partials (the key-range share of a context split across GPUs, each
 * holding a range of a sequence's keys; "diffbot/MiMo-V2.6-Flash-RL-FP8KV-
 * W4A8-2x-RTX-PRO-6000", What the kernels do: split-KV, here cut across key
 * ranges).  Computes, for every row of a verify-shaped call (max_q_len <= 16),
 * the attention above restricted to the keys key_lo[b] <= j < key_hi[b] of
 * its sequence, without the sink:
 *   out_part  fp32 [total_q, Hq, 128]: sum over those keys of p_j V_j / sum p_j
 *             (v_scale applied), 0 for a row that sees no key in the range
 *   lse_part  fp32 [total_q, Hq]: natural log-sum-exp of those keys' logits,
 *             -inf for a row that sees none
 *   key_lo, key_hi  int32 [batch] device arrays, or NULL for 0 / no bound
 * Only block-table entries of pages holding a key in the range are read, so
 * a caller holding part of a sequence may leave the others invalid.  The
 * workspace is the verify entry's: diffkv_attn_workspace_bytes(desc,
 * DIFFKV_ENTRY_VERIFY).  Other arguments, ownership and errors as for
 * attention; count_out counts the keys in range.  Partials of disjoint ranges
 * covering every visible key, merged by diffkv_attn_combine with the sinks,
 * give the attention output.
 */
int diffkv_attn_partial(const diffkv_attn_desc* desc, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                        const int32_t* q_lens, const int32_t* key_lo, const int32_t* key_hi,
                        int32_t window, float k_scale, float v_scale, float softmax_scale,
                        float* out_part, float* lse_part, int32_t* count_out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * Merge of context partials for `rows` = total_q * num_q_heads rows (row r is
 * query head r % num_q_heads):
 *   out_parts  fp32 [num_parts, rows, 128], lse_parts fp32 [num_parts, rows]
 *              (diffkv_attn_partial's outputs, stacked; -inf marks a part
 *              with no key for that row)
 *   sinks      fp32 [num_q_heads] or NULL, joining the merged denominator once
 *   out        bf16 [rows, 128]: sum_s w_s out_s / (sum_s w_s + e^(sink - M)),
 *              w_s = e^(lse_s - M), M = max(lse_s, sink); 0 if nothing is visible
 *   lse_out    fp32 [rows] (keys only) or NULL
 * num_parts in [1, 64] (DIFFKV_UNSUPPORTED beyond); rows a positive multiple
 * of num_q_heads.  Parts are summed in index order (deterministic).
 */
int diffkv_attn_combine(int32_t num_parts, int32_t rows, int32_t num_q_heads,
                        const float* out_parts, const float* lse_parts, const float* sinks,
                        void* out, float* lse_out, hipStream_t stream);

/*
 * Paged KV write: stores the new tokens' K and V rows into their cache slots,
 * the step before attention reads them ("diffbot/MiMo-V2.6-Flash-RL-FP8KV-
 * W4A8-2x-RTX-PRO-6000", intro: an E4M3 KV cache with per-tensor scales;
 * "sglang PR 32818": K and V in two caches of different row widths).
 *
 *   k_new        bf16 [total_q, Hkv, D_qk], packed by sequence like q above
 *   v_new        bf16 [total_q, Hkv, 128]
 *   k_cache, v_cache, block_table, seq_lens, q_lens: as for attention (the
 *                same descriptor serves both calls; num_q_heads is checked
 *                but not used)
 *   k_scale, v_scale  FP8 caches only: finite and > 0, else
 *                DIFFKV_INVALID_ARGUMENT; ignored for bf16 caches
 *
 * New token i of sequence b (position p = seq_lens[b] - q_lens[b] + i) goes
 * to slot p % P of page block_table[b][p / P], for every KV head.  A bf16
 * cache receives the rows bit for bit.  An FP8 cache receives, per value x,
 * the E4M3FN code of the fp32 quotient x / scale (correctly rounded
 * division), clamped to +-448 and rounded to nearest even; NaN becomes 0x7F
 * with the sign of the input, -0 becomes 0x80.  No other byte of either
 * cache changes.
 *
 * Same ownership and data preconditions as attention (the call only writes
 * the caches).  If two new tokens map to the same slot, which write lands is
 * unspecified.  Unlike the attention calls, a token whose position is
 * negative, whose page lies past block_table_stride or outside
 * [0, num_pages), or whose packed row is not below total_q, is skipped:
 * nothing is written for it.
 */
int diffkv_kv_write(const diffkv_attn_desc* desc, const void* k_new, const void* v_new,
                    void* k_cache, void* v_cache, const int32_t* block_table,
                    const int32_t* seq_lens, const int32_t* q_lens, float k_scale, float v_scale,
                    hipStream_t stream);

/* Bytes of workspace the entry needs for this descriptor (0 when none) on
 * the current device.  Host only: depends on the descriptor and the device's
 * compute-unit count (queried once per device and cached; 256, MI355X's
 * count, when no device can be queried).  A call on a stream of another
 * device with more compute units may need more (it then returns
 * DIFFKV_WORKSPACE_TOO_SMALL).  Returns 0 for an invalid descriptor (check
 * diffkv_attn_validate). */
size_t diffkv_attn_workspace_bytes(const diffkv_attn_desc* desc, int entry);

/* Synchronous check of a descriptor for an entry; host only, no HIP call. */
int diffkv_attn_validate(const diffkv_attn_desc* desc, int entry);

/* Upper bound on the key-axis chunks one (sequence, query tile) pair is cut
 * into for this descriptor and window (the kernels cut the keys on the
 * device from the actual lengths, in chunks that fit one resident round of
 * workgroups; this host-side bound sizes the merge): 1 when the keys are
 * not split (prefill, short windows), force_num_splits when that is set;
 * for mixed, the bound of its split-KV part; 0 for an invalid descriptor.
 * Host only; for the current device's compute-unit count. */
int diffkv_attn_num_splits(const diffkv_attn_desc* desc, int entry, int32_t window);

/* Debug builds only (the library compiled with -DDIFFKV_DEBUG, shipped as
 * libdiffkv_attn_debug.so).  Their kernels check the preconditions on device
 * data above (1 <= q_lens[b] <= seq_lens[b] <= max_seq_len, q_lens[b] <=
 * max_q_len, sum(q_lens) == total_q, every block-table entry read in
 * [0, num_pages)); a violation sets a bit in a device-wide word (1: a q_len,
 * 2: a seq_len, 4: a block-table entry, 8: the row total) and the offending
 * value is replaced by one that keeps every memory access in bounds, so the
 * call completes with a meaningless result rather than fault.  This call
 * enqueues on `stream` a copy of that word to the caller's device word
 * `flags` and clears it.  Release builds return DIFFKV_UNSUPPORTED and
 * enqueue nothing; NULL flags is DIFFKV_INVALID_ARGUMENT. */
int diffkv_attn_debug_flags(uint32_t* flags, hipStream_t stream);

/* Timeline builds only (the library compiled with -DDIFFKV_TIMELINE, shipped
 * as libdiffkv_attn_timeline.so; a measurement tool, not for production
 * calls).  Their split-KV kernels stamp the shader real-time counter (100
 * MHz) at eight points of each workgroup's work: 0 start, 1 lengths (and
 * the plan's totals) in, 2 own key range known, 3 first K/V data in (the
 * short-range pass: all of K), 4 first tile done (the short-range pass: its
 * products done), 5 last round of the tile loop, 6 epilogue, 7 output
 * stores issued.  A workgroup that finishes a chunk writes its eight stamps
 * to stamps[8 w .. 8 w + 7], w = blockIdx.y * gridDim.x + blockIdx.x, while
 * 8 w + 7 < entries, the stamps it did not pass as 0.  This call
 * registers the caller's device buffer (NULL with entries 0 turns the
 * writes off) for the current device, synchronously, so it must not be
 * captured into a graph; the buffer must stay valid while timed calls run.
 * Other builds return DIFFKV_UNSUPPORTED; exactly one of stamps == NULL and
 * entries == 0 is DIFFKV_INVALID_ARGUMENT. */
int diffkv_attn_timeline_buffer(uint64_t* stamps, size_t entries);

/* Static text for a status code. */
const char* diffkv_attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* DIFFKV_ATTN_H */
