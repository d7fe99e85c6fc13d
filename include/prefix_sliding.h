/*
 * prefix_sliding.h -- C ABI of the Prefix Sliding attention library (gfx950).
 *
 * Prefix Sliding: a query at absolute position p attends only to the pinned
 * prefix [0, L) and to the last W tokens (p-W, p], causally.  Source: blog
 * "Prefix Sliding 完全拆解" (pinghaoyang.com.cn), section
 * "核心机制：注意力掩码上的两个区间" (the allowed set A(i), the cap
 * L_total = L_prefix + W, warm-up, hidden tokens not kept).  Positions here
 * are 0-indexed; W counts the query itself, so a sequence never holds more
 * than L + W keys (100 + 4096 -> 4196, as the agihunt.info summary states).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer argument named *_cache, q, k, v, out, lse, workspace,
 *    block_table, prefix_len, pos, start_pos, seq_tokens, slot_pos, tiles,
 *    num_tiles is a DEVICE pointer.  Descriptors are HOST pointers, read
 *    during the call only.
 *  - The caller owns every buffer and the stream.  The library never
 *    allocates, frees or synchronises; work is enqueued on `stream` and runs
 *    asynchronously.  Calls on one stream run in order (append before the
 *    decode that reads the token).
 *  - Arguments the host can see are validated before anything is enqueued;
 *    on failure nothing is launched, the status says why and
 *    ps_last_error() returns a thread-local message.  Launch failures return
 *    PS_HIP_ERROR.  Faults in asynchronous work surface at the caller's next
 *    synchronisation.
 *  - Per-sequence values that live on the device (prefix_len, pos,
 *    start_pos, block_table entries) cannot be checked by the host.  A
 *    sequence whose values are out of range (prefix_len < 0, a position < 0,
 *    a slot at or beyond slot_capacity -- i.e. min(p+1, L+W) > slot_capacity
 *    -- or a page id outside [0, num_pages)) is never read or written out of
 *    bounds: such appends are dropped and its decode output rows are NaN.
 *    A ring of L + W <= slot_capacity slots serves any position; a window
 *    wider than the capacity (the full-attention comparator, W >= n) works
 *    while the sequence is shorter than the capacity.
 *  - Element tensors (caches, q, k, v, out, k_new, v_new, d_out, dq, dk, dv,
 *    score, workspace) are accessed with 16-byte vector loads and stores and
 *    must be 16-byte aligned; lse must be 4-byte aligned.  A misaligned
 *    pointer (e.g. a view at an odd storage offset) is PS_INVALID_ARGUMENT.
 *  - The library keeps no mutable global state; calls are reentrant.
 *
 * KV cache layout (owned by the caller, defined here)
 * ---------------------------------------------------
 * The cache of one layer is a set of 64-slot REGIONS, one per
 * (page or ring segment, KV head).  A region holds D*64 elements of K and
 * D*64 elements of V (elements are bf16 or f32, per ps_attn_desc.dtype):
 *    K region: row-major [64 slots][D]
 *    V region: 8 blocks of 8 slots, each block d-major: [8][D][8]
 *              (slot s, dim d at (s/8)*8*D + d*8 + s%8)
 * V is stored this way so that 8 consecutive slots of one dimension are 16
 * contiguous bytes: exactly one operand register of a bf16 MFMA that
 * contracts over keys.
 *  - Contiguous mode (page_size == 0): sequence s, KV head h, slot j lives in
 *    region ((s*Hkv + h) * slot_capacity/64 + j/64); i.e. the K cache is
 *    [num_seqs][Hkv][slot_capacity][D] and V is the same size.
 *  - Paged mode (page_size == 64): slot j of sequence s lives in page
 *    block_table[s*max_pages_per_seq + j/64]; page P, KV head h is region
 *    (P*Hkv + h); i.e. the K pool is [num_pages][Hkv][64][D].
 * Slots follow the ring map of Continue PE (blog section
 * "位置编码：Reset PE 还是 Continue PE？": every token keeps its absolute
 * position, cached keys are rotated once and reused):
 *    slot(n) = n                         if n < L
 *            = L + ((n - L) mod W)       otherwise,
 * so appending position n overwrites position n - W, the token that has just
 * left the window, and after warm-up slots [0, L+W) hold exactly A(p).  K is
 * stored already rotated (RoPE at its absolute position); V is not rotated.
 */
#ifndef PREFIX_SLIDING_H
#define PREFIX_SLIDING_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PS_ABI_VERSION 9

typedef enum {
  PS_OK = 0,
  PS_INVALID_ARGUMENT = 1,
  PS_UNSUPPORTED = 2,
  PS_WORKSPACE_TOO_SMALL = 3,
  PS_HIP_ERROR = 4
} ps_status;

typedef enum { PS_BF16 = 0, PS_F32 = 1 } ps_dtype;

/* Position encoding of the visible window (blog "Prefix Sliding 完全拆解",
 * section "位置编码：Reset PE 还是 Continue PE？").  Continue PE: every token
 * keeps its absolute position (the method's choice).  Reset PE (the ablated
 * alternative): the visible window tokens are renumbered to follow the prefix
 * directly, oldest first, and the query takes the last number,
 * min(p, prefix_len + W - 1).  Only ps_decode_attn accepts PS_PE_RESET: the
 * cache still holds keys rotated at their absolute positions, because
 * renumbering shifts every window key and the query by the same amount, which
 * leaves their rotary offsets unchanged -- so window keys are scored as under
 * Continue PE and only the prefix keys are scored against the query rotated at
 * its renumbered position (no key is re-rotated). */
/* PS_PE_RESET_RECOMPUTE computes the same Reset-PE attention the way the blog
 * describes its cost: ps_kv_append stores K un-rotated, and every
 * ps_decode_attn call first rotates each visible key at its renumbered
 * position (prefix slot j keeps j; the window token at absolute position n
 * becomes L + n - max(L, p - W + 1)) into a scratch copy in the workspace,
 * then runs the ordinary decode with the query at min(p, L + W - 1).
 * Contiguous caches only; decode only (other entry points return
 * PS_UNSUPPORTED).  It exists to measure what PS_PE_RESET avoids. */
typedef enum { PS_PE_CONTINUE = 0, PS_PE_RESET = 1, PS_PE_RESET_RECOMPUTE = 2 } ps_pe_mode;

/* Attention geometry.
 * num_q_heads % num_kv_heads == 0; query head h uses KV head
 * h / (num_q_heads/num_kv_heads) (consecutive heads share a KV head);
 * the group size must be <= 16.  head_dim is 64 or 128.
 * rope_theta > 0: rotate-half RoPE with inverse frequencies
 * rope_theta^(-2i/D), pairing dims (i, i + D/2), applied inside the library at
 * absolute positions (angle formed in double precision); 0: inputs are already
 * rotated.  softmax_scale > 0 multiplies q.k before the softmax. */
typedef struct {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;            /* ps_dtype: element type of q, k, v, caches, out */
  double rope_theta;
  float softmax_scale;
  int32_t pe_mode;          /* ps_pe_mode; 0 = Continue PE */
} ps_attn_desc;

/* Cache geometry.  window = W >= 1.  page_size 0 (contiguous) or 64 (paged).
 * slot_capacity: slots per (sequence, KV head), a multiple of 64; a
 * sequence at position p uses slots [0, min(p+1, prefix_len + W)).  Paged mode also needs
 * max_pages_per_seq == slot_capacity/64 (row length of block_table) and
 * num_pages (pages in the pool, bound for block_table entries). */
typedef struct {
  int32_t window;
  int32_t page_size;
  int32_t slot_capacity;
  int32_t max_pages_per_seq;
  int64_t num_pages;
} ps_cache_desc;

/* ps_kv_append -- write new tokens' K (rotated at their absolute position) and
 * V into their ring slots.  Blog "Prefix Sliding 完全拆解", mask section (hidden
 * tokens are not kept) and the Continue PE section (rotate once, reuse).
 *   k_new, v_new : [num_seqs][tokens_per_seq][Hkv][D], dtype of attn, raw K.
 *   start_pos    : [num_seqs] int64, absolute position of token 0.
 *   seq_tokens   : [num_seqs] int32 tokens actually present per sequence
 *                  (<= tokens_per_seq), or NULL for tokens_per_seq each.
 *   prefix_len   : [num_seqs] int32 L of each sequence.
 *   block_table  : paged mode [num_seqs][max_pages_per_seq] int32, else NULL.
 *   slot_pos     : NULL, or [num_seqs][slot_capacity] int32 that receives the
 *                  absolute position written into each slot (for checking).
 * Within one call a token at position j is written only if j < L or
 * j > p_last - W (p_last = the sequence's last position in the call): tokens
 * that the same call would already evict are skipped, so no two writes of a
 * call hit the same slot.  tokens_per_seq == 0 or num_seqs == 0 is a no-op.
 * With pe_mode PS_PE_RESET_RECOMPUTE the keys are stored un-rotated. */
ps_status ps_kv_append(const ps_attn_desc* attn, const ps_cache_desc* cache,
                       void* k_cache, void* v_cache, const int32_t* block_table,
                       const int32_t* prefix_len, const int64_t* start_pos,
                       const int32_t* seq_tokens, int32_t tokens_per_seq,
                       const void* k_new, const void* v_new, int32_t num_seqs,
                       int32_t* slot_pos, hipStream_t stream);

/* ps_decode_attn -- one decode query per sequence over its bounded cache.
 * Blog "Prefix Sliding 完全拆解", mask section (A(i); the per-token cost is
 * constant after warm-up) and section "Kernel 实现：两层级过滤" (only the
 * prefix and the window are read).
 *   q   : [num_seqs][Hq][D] raw (un-rotated) queries, dtype of attn.
 *   pos : [num_seqs] int64 absolute query position p; the cache must already
 *         hold position p (append first).  The query sees ring slots
 *         [0, min(p+1, L+W)), which are exactly A(p).
 *   out : [num_seqs][Hq][D], dtype of attn.
 *   num_splits : key-range splits per (sequence, KV head); 0 picks one from
 *         the device's CU count (ps_decode_num_splits).  Partial results are
 *         merged in a fixed order, so results are bitwise reproducible for a
 *         given split count.
 *   workspace : device scratch of at least
 *         ps_decode_workspace_size(attn, cache, num_seqs, num_splits) bytes. */
ps_status ps_decode_attn(const ps_attn_desc* attn, const ps_cache_desc* cache,
                         const void* k_cache, const void* v_cache, const int32_t* block_table,
                         const int32_t* prefix_len, const int64_t* pos,
                         const void* q, void* out, int32_t num_seqs, int32_t num_splits,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ps_decode_step -- one decode step: ps_kv_append of the token at pos
 * (k_new, v_new: [num_seqs][1][Hkv][D]) followed by ps_decode_attn at pos,
 * with the same arguments, rules and results: the ring contents are
 * bit-identical to those ps_kv_append writes, and the output is within the
 * decode tolerance of the two calls made in turn.  For bf16 and Continue PE it
 * is one launch: inside the decode kernel, the wave that will read the ring
 * chunk holding the token's slot rotates and stores the token while its
 * first loads are in flight, and issues its loads of that chunk only after
 * its stores have completed (an explicit wait when the chunk is among its
 * first two, otherwise the completion wait on an earlier chunk's loads, which
 * a wave's vector memory counter retires in issue order), so the token is read
 * back from memory like every other key.  Other dtypes and PE modes run the
 * two calls.  Every argument is validated before anything is enqueued.  Same
 * workspace as ps_decode_attn. */
ps_status ps_decode_step(const ps_attn_desc* attn, const ps_cache_desc* cache,
                         void* k_cache, void* v_cache, const int32_t* block_table,
                         const int32_t* prefix_len, const int64_t* pos, const void* q,
                         const void* k_new, const void* v_new, void* out, int32_t num_seqs,
                         int32_t num_splits, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* ps_decode_step_noalloc -- ps_decode_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same arguments minus the workspace, the same
 * rules and results.  The split partials go to a static device array inside
 * the library (ps_decode_noalloc_scratch_bytes() = 8 MiB per GPU, held until
 * the process ends); the call allocates nothing.  A call whose partials would
 * exceed it (ps_decode_workspace_size(...) > 8 MiB: e.g. more than about
 * 4,000 (sequence, split) pairs of 16 heads at head_dim 128, or
 * PS_PE_RESET_RECOMPUTE on a large cache) returns PS_WORKSPACE_TOO_SMALL
 * before anything is enqueued.  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (different streams, or host threads)
 * race and must be serialised by the caller.  The first call on a device
 * looks the array's device address up (hipGetSymbolAddress). */
ps_status ps_decode_step_noalloc(const ps_attn_desc* attn, const ps_cache_desc* cache,
                                 void* k_cache, void* v_cache, const int32_t* block_table,
                                 const int32_t* prefix_len, const int64_t* pos, const void* q,
                                 const void* k_new, const void* v_new, void* out, int32_t num_seqs,
                                 int32_t num_splits, hipStream_t stream);

/* Size of the static scratch array of ps_decode_step_noalloc, in bytes. */
size_t ps_decode_noalloc_scratch_bytes(void);

/* Split count ps_decode_attn uses for num_splits == 0 (queries the current
 * device; assumes 256 CUs when none is visible).  Returns >= 1, or 0 on
 * invalid arguments. */
int32_t ps_decode_num_splits(const ps_attn_desc* attn, const ps_cache_desc* cache, int32_t num_seqs);

/* Workspace bytes ps_decode_attn needs (num_splits 0: automatic).  With
 * pe_mode PS_PE_RESET_RECOMPUTE this includes the rotated copy of the keys
 * (num_seqs * Hkv * slot_capacity * head_dim elements) and a cos/sin table. */
size_t ps_decode_workspace_size(const ps_attn_desc* attn, const ps_cache_desc* cache,
                                int32_t num_seqs, int32_t num_splits);

/* ps_prefill_attn -- masked attention of a chunk of queries (truncated
 * backprop forward / prefill).  Blog "Prefix Sliding 完全拆解", sections
 * "Kernel 实现：两层级过滤" (tiles with no visible pair are skipped, element
 * masks only on tiles that are partly visible) and
 * "超长 rollouts 的反向传播：截断回传" (the trainer sees a chunk of the
 * trace behind the prefix).
 *   k, v : [batch][num_keys][Hkv][D] raw keys/values; key k has absolute
 *          position k for k < prefix_len and kv_start + (k - prefix_len)
 *          otherwise (kv_start >= prefix_len).
 *   q    : [batch][num_queries][Hq][D] raw queries; query t is key
 *          num_keys - num_queries + t (same position).  If the queries reach
 *          into the prefix (num_queries > num_keys - prefix_len), kv_start
 *          must equal prefix_len.
 *   out  : [batch][num_queries][Hq][D], dtype of attn.
 *   lse  : NULL or [batch][Hq][num_queries] float, natural-log sum of
 *          exp(scaled masked scores) per query row.
 *   workspace : >= ps_prefill_workspace_size(...) bytes (rotated keys and a
 *          rotation table for the query positions). */
ps_status ps_prefill_attn(const ps_attn_desc* attn, int32_t window, int32_t prefix_len,
                          int64_t kv_start, const void* q, const void* k, const void* v,
                          int32_t batch, int32_t num_queries, int32_t num_keys,
                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

size_t ps_prefill_workspace_size(const ps_attn_desc* attn, int32_t batch, int32_t num_queries,
                                 int32_t num_keys);

/* ps_heavy_decode_step -- one decode step with prefix + heavy hitters +
 * window.  Blog "Prefix Sliding 完全拆解", section comparing the method with
 * H2O: H2O keeps the tokens that have drawn the most attention (it looks
 * back), Prefix Sliding pins the prefix (it looks ahead); the two can be
 * stacked.  The pages give no algorithm; the rule implemented:
 *   - per (sequence, KV head), heavy_slots = H cache slots right after the
 *     window's ring slots: slots [0, L) prefix, [L, L+W) window, [L+W, L+W+H)
 *     heavy hitters, so L + W + H <= slot_capacity for every sequence;
 *   - a token's score is the softmax attention it has received while cached,
 *     summed over the query heads of its KV head;
 *   - at step p the token p - W leaves the window; it takes the next free
 *     heavy slot, or replaces the member with the smallest score (ties: the
 *     oldest position) if its own score is strictly larger, else it is dropped;
 *   - then the token p is appended (as ps_kv_append), the query at p attends
 *     to prefix + heavy set + window, and every visible non-prefix token adds
 *     the attention it just received to its score.
 * Arguments as ps_kv_append (k_new, v_new: [num_seqs][1][Hkv][D], the token
 * at pos) and ps_decode_attn (q, out, pos, num_splits, workspace), plus the
 * caller-owned state, zeroed when a sequence starts:
 *   score       : [num_seqs][Hkv][slot_capacity] float, 0 initially;
 *   heavy_count : [num_seqs][Hkv] int32, 0 initially;
 *   heavy_pos   : [num_seqs][Hkv][heavy_slots] int64 positions of the heavy
 *                 members (entries past heavy_count are unspecified).
 * Steps must be issued for consecutive positions of a sequence (the
 * admission at p needs the scores accumulated up to p - 1).  workspace:
 * >= ps_heavy_workspace_size(...) bytes (may be 0, then workspace may be
 * NULL: bf16 with one split whose per-slot statistics fit the kernel's LDS).
 * Continue PE only. */
ps_status ps_heavy_decode_step(const ps_attn_desc* attn, const ps_cache_desc* cache,
                               int32_t heavy_slots, void* k_cache, void* v_cache,
                               const int32_t* block_table, const int32_t* prefix_len,
                               const int64_t* pos, const void* q, const void* k_new,
                               const void* v_new, void* out, int32_t num_seqs, float* score,
                               int32_t* heavy_count, int64_t* heavy_pos, int32_t num_splits,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t ps_heavy_workspace_size(const ps_attn_desc* attn, const ps_cache_desc* cache,
                               int32_t num_seqs, int32_t num_splits);

/* ps_prefill_attn_backward -- gradients of ps_prefill_attn for the raw
 * inputs: dq, dk, dv from the upstream gradient d_out.  Blog "Prefix Sliding
 * 完全拆解", section "超长 rollouts 的反向传播：截断回传": the trainer receives
 * the last 4W tokens of a trace and back-propagates through the same masked
 * attention (its loss mask on the last W tokens only decides which rows of
 * d_out are non-zero); section "Kernel 实现：两层级过滤": the same tile
 * skipping applies.
 *   window, prefix_len, kv_start, q, k, v, batch, num_queries, num_keys :
 *          exactly as given to ps_prefill_attn.
 *   out  : the forward output [batch][num_queries][Hq][D].
 *   d_out: upstream gradient, same layout and dtype.
 *   lse  : the forward's LSE [batch][Hq][num_queries] (required).
 *   dq   : [batch][num_queries][Hq][D]; dk, dv : [batch][num_keys][Hkv][D];
 *          dtype of attn; fully overwritten (keys no query sees get zeros).
 *   workspace : >= ps_prefill_backward_workspace_size(...) bytes.  In bf16,
 *          when it also holds ps_prefill_backward_ds_workspace_size(...)
 *          more bytes, the dk/dv pass keeps its dS tiles there and the dq
 *          pass reads them instead of forming S and dP again (same
 *          arithmetic, one product instead of three); otherwise dq
 *          recomputes them.  The two paths may differ in the last bit of dq
 *          (fp32 sums in another order); dk and dv are the same.
 * Deterministic: every output row has exactly one writer (no atomics). */
ps_status ps_prefill_attn_backward(const ps_attn_desc* attn, int32_t window, int32_t prefix_len,
                                   int64_t kv_start, const void* q, const void* k, const void* v,
                                   const void* out, const void* d_out, const float* lse,
                                   int32_t batch, int32_t num_queries, int32_t num_keys,
                                   void* dq, void* dk, void* dv, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

size_t ps_prefill_backward_workspace_size(const ps_attn_desc* attn, int32_t batch,
                                          int32_t num_queries, int32_t num_keys);

/* Extra workspace bytes (beyond ps_prefill_backward_workspace_size's) with
 * which the bf16 backward keeps its dS tiles for the dq pass: one 128-key x
 * 64-query bf16 tile (16 KB) per query head, 64-query block and 128-key tile
 * of the block's walk, i.e. batch * Hq * ceil(num_queries / 64) * slots *
 * 16384 bytes, slots the longest walk (the pinned-key tiles, then the window
 * band: about (W + 64) / 128 + 2 tiles when the prefix fits one tile).  0 for
 * fp32 or invalid arguments (the dq pass then recomputes). */
size_t ps_prefill_backward_ds_workspace_size(const ps_attn_desc* attn, int32_t window,
                                             int32_t prefix_len, int64_t kv_start, int32_t batch,
                                             int32_t num_queries, int32_t num_keys);

/* ps_chunk_prefill_attn -- a chunk of new tokens continues cached traces:
 * attention of the chunk's queries over each sequence's ring plus the chunk
 * itself, after which the chunk joins the ring.  Blog "Prefix Sliding
 * 完全拆解": section "核心机制：注意力掩码上的两个区间" (A(i) for every
 * query; the ring keeps only prefix and window), the paged fixed-cap memory
 * remark that closes that section, and the multi-turn / tool-output case of
 * its limitations section (long external content poured into a live trace).
 *   prefix_len, start_pos : [num_seqs] device int32 / int64.  Sequence s
 *          holds positions [0, P) in its ring (P = start_pos[s], appended
 *          earlier through ps_kv_append / this call); the chunk is positions
 *          [P, P + chunk_len).
 *   q, k_new, v_new : [num_seqs][chunk_len][H][D] raw chunk queries / keys /
 *          values (H = Hq for q, Hkv for k_new and v_new), dtype of attn.
 *   out  : [num_seqs][chunk_len][Hq][D]; query t (position P + t) sees every
 *          visible key: ring keys below P and chunk keys up to itself.
 *   lse  : NULL or [num_seqs][Hq][chunk_len] float (as ps_prefill_attn).
 *   slot_pos : NULL or the ps_kv_append sidecar, updated by the append.
 *   workspace : >= ps_chunk_prefill_workspace_size(...) bytes.
 * Order: every chunk query reads the ring before any chunk token is written
 * into it (a chunk token may reuse the slot of a window key an earlier chunk
 * query still needs); both steps are enqueued on `stream`.
 * Device values that cannot be served -- negative L or P, or
 * min(P, L + W) > slot_capacity -- give NaN rows for that sequence (its
 * appends follow the ps_kv_append rules); a ring page outside the pool gives
 * NaN rows for the queries that see it. */
ps_status ps_chunk_prefill_attn(const ps_attn_desc* attn, const ps_cache_desc* cache,
                                void* k_cache, void* v_cache, const int32_t* block_table,
                                const int32_t* prefix_len, const int64_t* start_pos,
                                int32_t chunk_len, const void* q, const void* k_new,
                                const void* v_new, int32_t num_seqs, void* out, float* lse,
                                int32_t* slot_pos, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Workspace bytes ps_chunk_prefill_attn needs (0 on invalid arguments). */
size_t ps_chunk_prefill_workspace_size(const ps_attn_desc* attn, const ps_cache_desc* cache,
                                       int32_t num_seqs, int32_t chunk_len);

/* Tile shape (BM queries x BN keys) ps_prefill_attn uses for this geometry. */
ps_status ps_prefill_tile_shape(const ps_attn_desc* attn, int32_t* block_m, int32_t* block_n);

/* ps_prefill_plan -- the tile list ps_prefill_attn executes, for checking:
 * the attention kernel's walk itself (the same scheduling functions), which
 * visits exactly the (q_tile, k_tile) of the BM x BN grid holding at least one
 * visible (query, key) pair, sorted by q_tile then k_tile, as int32 triples
 * (q_tile, k_tile, kind) with kind 1 = every pair of the full BM x BN tile
 * exists and is visible (no element mask), 2 = partial (masked).  tiles is
 * [max_tiles][3]; *num_tiles receives the total count even when it exceeds
 * max_tiles (then only max_tiles triples are written).  Same geometry rules
 * as ps_prefill_attn. */
ps_status ps_prefill_plan(const ps_attn_desc* attn, int32_t window, int32_t prefix_len,
                          int64_t kv_start, int32_t num_queries, int32_t num_keys,
                          int32_t* tiles, int32_t max_tiles, int32_t* num_tiles,
                          hipStream_t stream);

/* ps_read_probe -- measurement helper, not part of the method: reads `bytes`
 * of device memory at src once (16-byte non-temporal loads, grid-stride over
 * the whole GPU) and stores the XOR of all its 32-bit words in *checksum
 * (device memory; 0 for bytes == 0).  Timed around a large buffer it gives the
 * HBM read bandwidth this GPU actually sustains, the measured ceiling the
 * decode kernel is reported against next to the published 8 TB/s.  src and
 * bytes must be 16-byte aligned, bytes <= 2^40; PS_INVALID_ARGUMENT otherwise,
 * before anything is launched. */
ps_status ps_read_probe(const void* src, size_t bytes, uint32_t* checksum, hipStream_t stream);

const char* ps_last_error(void);
const char* ps_status_string(ps_status status);
int32_t ps_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PREFIX_SLIDING_H */
