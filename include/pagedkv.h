/*
 * pagedkv.h -- C ABI of libpagedkv.so: attention over a block-paged KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed comes from the mlx-node documentation pages on its paged
 * KV cache and on performance:
 *   - the paged-cache doc, component table: per-layer K and V pools of
 *     fixed-size blocks (LayerKVPool), a block allocator with per-block
 *     refcounts, LRU eviction and a prefix table (BlockAllocator), and the
 *     per-request lifecycle reset -> find cached prefix -> allocate suffix
 *     blocks -> record tokens -> register full blocks for reuse -> release;
 *   - the paged-cache doc, hybrid coordinator paragraph: sliding-window
 *     groups keep absolute table width and map blocks wholly outside the
 *     window to a shared null sentinel; KV-shared layers alias their anchor;
 *   - the perf doc, paged-attention knobs table: a native paged K/V write, a
 *     decode gather through the pages (sliding groups from their first live
 *     block), batched multi-row paged decode, and the prefill chunk size;
 *   - the perf doc, attention-partitions paragraph: partitioned decode whose
 *     partials are combined by a reducer, extra empty partitions adding exact
 *     zeros.
 *
 * General conventions
 *   - Every function returns an int32 status: PAGED_OK (0) or a negative
 *     PAGED_ERR_* code. paged_last_error() returns a thread-local message for
 *     the last failure on the calling thread. No C++ exception crosses the ABI.
 *   - Device memory is owned by the caller (pools, inputs, outputs, decode
 *     workspace). The library never allocates or frees device memory and never
 *     synchronizes a stream, except paged_trace_query (see there).
 *   - Device work is enqueued on the caller's stream (a hipStream_t passed as
 *     void*; NULL = the null stream). Argument errors are detected on the host
 *     before anything is enqueued; nothing is enqueued when a call fails.
 *     Device-side faults surface at the caller's next synchronization.
 *   - Device pointers must be 16-byte aligned. Table and length contents live
 *     on the device and are not read by the host; the kernels never dereference
 *     a physical block id outside [1, num_blocks) nor a table column outside
 *     [0, max_blocks_per_seq). A key whose table entry is 0, out of range or
 *     past the table's width is absent: attention gives it weight zero (a
 *     query whose keys are all absent gets zeros) and the gather leaves its
 *     output rows untouched. Well-formed tables (the allocator's) never map
 *     an attended position to such an entry.
 *   - Pool layout: pool[num_blocks][num_kv_heads][block_size][head_dim],
 *     K and V in two separate buffers, element type given by `dtype`.
 *     Block 0 is the null sentinel shared by every sliding table: no kernel
 *     reads or writes it (a write slot inside block 0 counts as padding).
 *   - A slot is physical_block * block_size + offset (int64); slot < 0 means
 *     padding.
 *   - head_dim in {64, 128, 256, 512} (512: bf16 or FP8 pools, not float32);
 *     block_size a power of two in [8, 64];
 *     num_q_heads a multiple of num_kv_heads (query head h reads KV head
 *     h / (num_q_heads / num_kv_heads)).
 *   - The allocator is host-only C++, not thread-safe (one allocator per pool,
 *     i.e. per cache group; callers serialize access to one handle).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PAGEDKV_ABI_VERSION 2

enum {
  PAGED_OK = 0,
  PAGED_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size or geometry */
  PAGED_ERR_DTYPE = -2,       /* dtype not supported by this entry point */
  PAGED_ERR_NO_BLOCKS = -3,   /* allocator exhausted; nothing was changed */
  PAGED_ERR_CAPACITY = -4,    /* caller buffer too small / position not reserved */
  PAGED_ERR_STATE = -5,       /* unknown or duplicate sequence, bad lifecycle order */
  PAGED_ERR_HIP = -6          /* HIP runtime error (launch, device query) */
};

/* Element types. PAGED_FP8_E4M3 is the FP8 KV-cache format (perf doc,
 * quantization table: FP8 KV cache row, per-layer scales): OCP E4M3 codes
 * (bias 7, max 448, 0x7F/0xFF NaN); a stored code c stands for scale * c with
 * one K scale and one V scale per layer pool. */
enum { PAGED_F32 = 0, PAGED_BF16 = 1, PAGED_FP8_E4M3 = 2 };

/* Returns PAGEDKV_ABI_VERSION. */
int32_t paged_abi_version(void);

/* Message for the last failing call on this thread ("" if none). The pointer
 * stays valid until the next library call on the same thread. */
const char* paged_last_error(void);

/* ----------------------------------------------------------------------
 * Device entry points
 * -------------------------------------------------------------------- */

/* Slot-mapped KV write (perf doc, paged-attention knobs table: native paged
 * K/V write); dtype PAGED_F32, PAGED_BF16, or PAGED_FP8_E4M3 to copy codes
 * that are already quantized (paged_kv_write_fp8 quantizes). For every t in
 * [0, num_tokens) with
 * block_size <= slot_mapping[t] < num_blocks * block_size:
 *   k_pool[slot / block_size][h][slot % block_size][:] = new_k[t][h][:]
 * for every KV head h, and the same for V. Tokens with a negative slot, a
 * slot inside block 0 (the null sentinel) or an out-of-range slot write
 * nothing. Bytes are copied unchanged.
 *   k_pool, v_pool : device, [num_blocks][num_kv_heads][block_size][head_dim]
 *   new_k, new_v   : device, [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping   : device, int64 [num_tokens]
 * Two tokens mapping to the same slot race (the result is one of them).
 * num_tokens == 0 enqueues nothing and succeeds. */
int32_t paged_kv_write(void* k_pool, void* v_pool, const void* new_k, const void* new_v,
                       const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                       int32_t dtype, void* stream);

/* Quantizing KV write into FP8 pools (perf doc, quantization table: FP8 KV
 * cache with per-layer scales). As paged_kv_write, but each element x of
 * new_k (new_v) is stored as the E4M3 code of x / k_scale (x / v_scale):
 * the division in float32 (correctly rounded), then the nearest E4M3 value
 * with ties to the even code, magnitudes above 448 saturated to 448.
 *   k_pool, v_pool : device, uint8 codes [num_blocks][num_kv_heads][block_size][head_dim]
 *   new_k, new_v   : device, src_dtype (PAGED_BF16 or PAGED_F32),
 *                    [num_tokens][num_kv_heads][head_dim], finite
 *   k_scale, v_scale : finite, > 0
 * Errors as paged_kv_write; PAGED_ERR_DTYPE for another src_dtype. */
int32_t paged_kv_write_fp8(void* k_pool, void* v_pool, const void* new_k, const void* new_v,
                           const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                           int32_t src_dtype, float k_scale, float v_scale, void* stream);

/* Gather the attended positions of each row into contiguous buffers (perf doc,
 * paged-attention knobs table: the synchronous decode gather reads the pages a
 * row attends to, sliding groups from their first live block). A diagnostic
 * and test entry point: attention reads the pool in place. For row b with
 * n = seq_lens[b] and lo = (sliding_window > 0 ? max(0, n - sliding_window) : 0):
 *   out_k[out_offsets[b] + (p - lo)][h][:] = k_pool[bt[b][p / bs]][h][p % bs][:]
 * for p in [lo, n), every head h; the same for V.
 *   block_tables : device, int32 [batch][max_blocks_per_seq]
 *   seq_lens     : device, int32 [batch], each in [0, max_seq_len]
 *   out_offsets  : device, int64 [batch] (row start in out, in tokens)
 *   out_k, out_v : device, [sum of spans][num_kv_heads][head_dim]
 * Elements are copied as bytes: dtype PAGED_F32, PAGED_BF16 or PAGED_FP8_E4M3
 * (codes). */
int32_t paged_kv_gather(void* out_k, void* out_v, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* seq_lens, const int64_t* out_offsets, int32_t batch,
                        int32_t max_seq_len, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t num_blocks, int32_t sliding_window,
                        int32_t dtype, void* stream);

/* Partition size (tokens per split-K partition) that paged_attn_decode uses
 * when called with partition_tokens == 0, for these arguments and dtype.
 * With G = num_q_heads / num_kv_heads, span = max_seq_len (with a window:
 * min(max_seq_len, sliding_window + block_size - 1)) and CUs = the device's
 * compute units:
 *   bf16 and FP8 pools: a workgroup is 4 waves streaming 16-token stages over
 *     GT = the largest divisor of G up to 16 query heads; pairs = batch *
 *     num_kv_heads * (G / GT); wave slots = CUs * (4 at head_dim >= 256, 12
 *     for FP8 pools up to head_dim 128, else 8); s = ceil(pairs *
 *     ceil(span / 16) / wave slots) rounded up to a power of two (at least 1);
 *     partition = max(max(16, block_size), min(65536, 64 * s)).
 *   fp32 pools: GT = the largest of 4, 2, 1 dividing G; the largest power of
 *     two c in [64, 1024] with pairs * ceil(span / c) >= 4 * CUs (else 64), at
 *     least block_size.
 * The workspace then holds batch * num_q_heads * ceil(span / partition) *
 * (head_dim + 2) floats, none when that ceiling is 1. A pure function of the
 * arguments and the CU count, so a given call reproduces exactly. Needs a
 * device (PAGED_ERR_HIP otherwise). */
int32_t paged_attn_decode_partition_tokens(int32_t batch, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t block_size, int32_t max_seq_len,
                                           int32_t sliding_window, int32_t dtype,
                                           int32_t* partition_tokens);

/* Bytes of device workspace paged_attn_decode needs for these arguments and
 * dtype (0 when every row fits one partition: the kernel then writes the
 * output directly and no reduce pass runs). partition_tokens == 0 asks for
 * the library rule above (needs a device). */
int32_t paged_attn_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t max_seq_len,
                                          int32_t sliding_window, int32_t partition_tokens,
                                          int32_t dtype, size_t* bytes);

/* Batched GQA decode over the paged cache: one query token per row, the row's
 * newest (its K/V already written), attending to positions
 * [lo, n) with n = seq_lens[b], lo = max(0, n - sliding_window) when
 * sliding_window > 0 else 0 (perf doc, knobs table: batched paged decode;
 * paged-cache doc, hybrid coordinator paragraph: sliding groups and the null
 * sentinel). Per query head h (KV head h / G), with scale finite and > 0
 * (PAGED_ERR_INVALID_ARG otherwise):
 *   o[b][h] = sum_t softmax_t(scale * q[b][h] . K[t]) V[t]
 * A row with n == 0 gives zeros. Long rows are split into partitions of
 * `partition_tokens` positions counted from the first live block of the row
 * (the block holding lo); each partition produces float32 (max, sum, acc)
 * partials in `workspace`, which a second kernel combines in partition order
 * (deterministic, no atomics; perf doc, attention-partitions paragraph).
 *   out, q         : device, [batch][num_q_heads][head_dim], element type dtype
 *   k_pool, v_pool : device, pool layout above, same dtype
 *   block_tables   : device, int32 [batch][max_blocks_per_seq]
 *   seq_lens       : device, int32 [batch], each in [0, max_seq_len]
 *   partition_tokens: 0 = library rule, else a multiple of block_size in [16, 65536];
 *                  ceil(span / partition_tokens) (span = max_seq_len, or the window
 *                  plus block_size - 1 with a window) must be at most 65535,
 *                  and the span at most 2^30 tokens (PAGED_ERR_INVALID_ARG otherwise)
 *   workspace      : device, >= paged_attn_decode_workspace_bytes(...) bytes
 * For a KV-shared layer pass the anchor layer's pools and tables; for a
 * sliding layer pass its own pool, tables and window. */
int32_t paged_attn_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, float scale, int32_t sliding_window,
                          int32_t partition_tokens, int32_t max_seq_len, void* workspace,
                          size_t workspace_bytes, int32_t dtype, void* stream);

/* paged_attn_decode over FP8 pools: K[t] = k_scale * E4M3(k code), V[t] =
 * v_scale * E4M3(v code); q and out bf16. Same partitions, workspace (query
 * it with dtype PAGED_FP8_E4M3) and errors as paged_attn_decode.
 *   k_scale, v_scale : finite, > 0, the scales the pools were written with */
int32_t paged_attn_decode_fp8(void* out, const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, float scale, float k_scale, float v_scale,
                              int32_t sliding_window, int32_t partition_tokens,
                              int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                              void* stream);

/* paged_attn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * same kernels and partitions as paged_attn_decode (f32 or bf16 pools), with
 * the split-K partials in a device array the library holds per GPU (16 MiB,
 * kept until the process ends) instead of a caller workspace; the caller
 * still passes inputs and outputs. Nothing is allocated by the call.
 * PAGED_ERR_CAPACITY when the partials need more than 16 MiB
 * (paged_attn_decode_workspace_bytes gives the need for the same arguments).
 * The partials need no clearing between calls: every partition a row uses is
 * written before the reduce reads it. Every call on one GPU shares that
 * array: calls that overlap on one GPU (several streams, several host
 * threads) race on it and give wrong results. */
int32_t paged_attn_decode_noalloc(void* out, const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, float scale, int32_t sliding_window,
                                  int32_t partition_tokens, int32_t max_seq_len, int32_t dtype,
                                  void* stream);

/* Chunked-prefill attention over a cached paged prefix (perf doc, knobs table:
 * prefill chunk size; the paged-attention bridge for prefill over a cache hit
 * that reads K/V through the pages). Row b owns query rows
 * [cu_q_lens[b], cu_q_lens[b+1]) of q (C of them) and has
 * seq_lens[b] = P + C cached tokens, the chunk's own K/V already written.
 * Query i of the chunk sits at position a = P + i and attends to keys
 * [lo, a], lo = max(0, a - sliding_window + 1) when sliding_window > 0 else 0
 * (causal inside the chunk). bf16 only; the products run on MFMA with float32
 * accumulation, probabilities rounded to bf16 for the P.V product. scale must
 * be finite and > 0 (PAGED_ERR_INVALID_ARG otherwise); q, K and V must be
 * finite (NaN inputs give unspecified results).
 *   out, q       : device bf16, [total_q][num_q_heads][head_dim]
 *   cu_q_lens    : device int32 [batch + 1], cu_q_lens[0] = 0, nondecreasing,
 *                  cu_q_lens[batch] = total_q, each chunk <= max_q_len
 *   seq_lens     : device int32 [batch], seq_lens[b] >= chunk length of b
 *   workspace    : NULL, or device memory (16-byte aligned, caller-owned, not
 *                  read before it is written) of at least
 *                  paged_attn_prefill_chunk_workspace_bytes(...) bytes for the
 *                  same shapes. With NULL one workgroup covers each tile of
 *                  query rows over its whole key range. With a workspace, when
 *                  the query tiles are fewer than the device's compute units
 *                  (few rows or few heads, e.g. one GPU's share of KV heads),
 *                  the key range of every tile is cut into S near-equal parts
 *                  (S the smallest power of two up to 16 that gives every CU a
 *                  workgroup), each part's unnormalised output and (max, sum)
 *                  go to the workspace and a second kernel combines the S
 *                  parts of each (query, head) like the decode reduce. The
 *                  result is the same attention up to float rounding.
 *                  PAGED_ERR_INVALID_ARG when it is misaligned or too small. */
int32_t paged_attn_prefill_chunk(void* out, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
                                 const int32_t* seq_lens, int32_t batch, int32_t total_q,
                                 int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 float scale, int32_t sliding_window, void* workspace,
                                 size_t workspace_bytes, int32_t dtype, void* stream);

/* Bytes of workspace paged_attn_prefill_chunk (and _fp8) use for these shapes
 * on the current device (0: no key split, the workspace may be NULL). Needs a
 * device (the split depends on its compute-unit count): PAGED_ERR_HIP without one. */
int32_t paged_attn_prefill_chunk_workspace_bytes(int32_t batch, int32_t total_q,
                                                 int32_t max_q_len, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim,
                                                 size_t* bytes);

/* paged_attn_prefill_chunk over FP8 pools (K, V as in paged_attn_decode_fp8);
 * q and out bf16. Same arguments and errors otherwise. */
int32_t paged_attn_prefill_chunk_fp8(void* out, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
                                     const int32_t* seq_lens, int32_t batch, int32_t total_q,
                                     int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     float scale, float k_scale, float v_scale,
                                     int32_t sliding_window, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* One continuous-batching step over one layer (batching-perf-path doc,
 * current state: chunked prefill of joining requests interleaved with the
 * running decode rows). Rows [0, num_decode_rows) are decode rows with one
 * query each (cu_q_lens[b] == b for b <= num_decode_rows: query b is row b's
 * newest position); rows [num_decode_rows, batch) are prefill chunks. The
 * result is the attention paged_attn_prefill_chunk computes over all rows (a
 * decode row is a chunk of one), up to float rounding; the decode rows run
 * through the split-K decode kernels on `stream`, the chunk rows through the
 * prefill kernel (no key split: the decode fills the other CUs) on a second
 * stream the library keeps per device, so both run at once; `stream` waits
 * for both before anything enqueued after the call. The first call on a
 * device creates that stream and two events (keep it outside graph capture);
 * afterwards calls are capturable.
 *   out, q         : device bf16, [total_q][num_q_heads][head_dim]
 *   k_pool, v_pool : device, kv_dtype PAGED_BF16 (k_scale = v_scale = 1) or
 *                    PAGED_FP8_E4M3 (values k_scale * code, v_scale * code)
 *   block_tables   : device int32 [batch][max_blocks_per_seq]
 *   cu_q_lens      : device int32 [batch + 1], as for paged_attn_prefill_chunk
 *   seq_lens       : device int32 [batch]; decode rows' at most max_seq_len
 *   max_q_len      : bound on the chunk rows' query counts
 *   partition_tokens, max_seq_len, workspace: as for paged_attn_decode with
 *                    batch = num_decode_rows (size the workspace with
 *                    paged_attn_decode_workspace_bytes(num_decode_rows, ...))
 * Errors: those of both entry points, checked before anything is enqueued. */
int32_t paged_attn_mixed(void* out, const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* cu_q_lens, const int32_t* seq_lens, int32_t batch,
                         int32_t num_decode_rows, int32_t total_q, int32_t max_q_len,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, float scale, float k_scale,
                         float v_scale, int32_t sliding_window, int32_t partition_tokens,
                         int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                         int32_t kv_dtype, void* stream);

/* ----------------------------------------------------------------------
 * Kernel timing (HIP events around every launch, on the launch's stream)
 * -------------------------------------------------------------------- */

enum {
  PAGED_KERNEL_KV_WRITE = 0,
  PAGED_KERNEL_KV_GATHER = 1,
  PAGED_KERNEL_DECODE_PARTIAL = 2,
  PAGED_KERNEL_DECODE_REDUCE = 3,
  PAGED_KERNEL_PREFILL = 4,
  PAGED_KERNEL_PREFILL_REDUCE = 5,
  PAGED_KERNEL_COUNT = 6
};

/* on != 0: from now on, every launch records a start and an end event on its
 * stream (events are created lazily; no device memory is allocated). Launches
 * on a stream that is being captured into a graph record nothing. */
int32_t paged_trace_enable(int32_t on);
/* Drop all recorded launches. */
int32_t paged_trace_reset(void);
/* Wait for the recorded events of `kernel` and return the sum of their
 * elapsed times and the number of launches. Synchronizes those events. The
 * events are stamped at the kernel's own start and end (hipExtLaunchKernel),
 * so host launch overhead is not included. */
int32_t paged_trace_query(int32_t kernel, double* total_ms, int64_t* launches);
/* Per-launch durations of `kernel` in launch order: ms[i] for the first
 * min(capacity, *launches) launches; *launches = launches recorded. */
int32_t paged_trace_durations(int32_t kernel, double* ms, int64_t capacity, int64_t* launches);

/* ----------------------------------------------------------------------
 * Host block allocator (paged-cache doc, component table: BlockAllocator)
 *
 * Policy: block 0 is the null sentinel (never handed out). Free blocks form a
 * FIFO, initially `free_order` (a permutation of 1..num_blocks-1 drawn by the
 * caller; NULL = ascending); allocation pops the head, freed unpublished
 * blocks join the tail. The caller passes the permutation itself rather than
 * a seed: the physical placement then follows whatever generator the caller
 * uses (the test and benchmark inputs draw it with numpy's default_rng), and
 * the library and any reference allocator agree on it without both having
 * to implement one generator's permutation algorithm. Publishing enters a full block in the prefix table
 * under the exact key (domain, parent chain id, the block's token ids) and
 * gives it a fresh chain id (never reused). A published block whose refcount
 * reaches 0 joins the LRU tail and stays matchable; when the free list is
 * empty, allocation evicts the LRU head (dropping its key). Reservations are
 * all or nothing. Release walks a table from its last entry to its first.
 * -------------------------------------------------------------------- */

typedef struct paged_alloc paged_alloc;

/* num_blocks >= 2, block_size >= 1; free_order NULL or num_blocks-1 int32
 * entries forming a permutation of 1..num_blocks-1. *out owns the handle. */
int32_t paged_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                           paged_alloc** out);
int32_t paged_alloc_destroy(paged_alloc* a);
/* Add blocks num_blocks..new_num_blocks-1 to the free tail in the order given
 * (NULL = ascending); the caller grows its device pools to match first
 * (paged-cache doc, pool-sizing section: grow before evicting). */
int32_t paged_alloc_grow(paged_alloc* a, int32_t new_num_blocks, const int32_t* new_order);
/* Ceiling for paged_seq_reserve_or_grow (paged-cache doc, pool-sizing section:
 * the maximum pool size). The default is the pool's size at creation (a fixed
 * pool, which never asks to grow); paged_alloc_grow raises it to the new size
 * when that is larger. PAGED_ERR_INVALID_ARG below the current block count. */
int32_t paged_alloc_set_max_blocks(paged_alloc* a, int32_t max_blocks);
int32_t paged_alloc_num_blocks(const paged_alloc* a, int32_t* num_blocks);
int32_t paged_alloc_num_free(const paged_alloc* a, int32_t* free_blocks,
                             int32_t* evictable_blocks);

/* reset_for_new_request: a new, empty sequence. PAGED_ERR_STATE if it exists. */
int32_t paged_seq_add(paged_alloc* a, int64_t seq_id);
/* find_cached_prefix: share the longest published chain of full blocks that
 * prefixes tokens[0..n) in `domain` (refcount + 1 each; an evictable block
 * leaves the LRU queue). The sequence must hold no blocks. *cached_tokens =
 * matched blocks * block_size. Callers that must recompute the last prompt
 * token pass n = prompt length - 1. */
int32_t paged_seq_match_prefix(paged_alloc* a, int64_t seq_id, const int32_t* tokens,
                               int32_t n, uint64_t domain, int32_t* cached_tokens);
/* Fork: the empty sequence dst references src's first num_blocks full blocks. */
int32_t paged_seq_share_prefix(paged_alloc* a, int64_t dst_seq, int64_t src_seq,
                               int32_t num_blocks);
/* allocate_suffix_blocks: grow the table to ceil(total_tokens / block_size)
 * entries. PAGED_ERR_NO_BLOCKS (nothing changed) if free + evictable is short. */
int32_t paged_seq_reserve(paged_alloc* a, int64_t seq_id, int32_t total_tokens);
/* allocate_suffix_blocks with grow-on-demand (paged-cache doc, pool-sizing
 * section: a reservation that outruns free + evictable blocks grows the pool
 * before evicting; one grow, then one retry). With needed = the new blocks the
 * reservation takes and cur = the pool's block count:
 *   - needed <= free + evictable: reserved as by paged_seq_reserve
 *     (free blocks first, then LRU eviction); *grow_to = 0;
 *   - else, cur < max: nothing changes and *grow_to =
 *     min(max, max(2 * cur, cur + needed)); the caller grows its device pools
 *     to *grow_to blocks, calls paged_alloc_grow, then retries once with
 *     paged_seq_reserve (which reserves, evicting as needed, or fails);
 *   - else PAGED_ERR_NO_BLOCKS (nothing changed). */
int32_t paged_seq_reserve_or_grow(paged_alloc* a, int64_t seq_id, int32_t total_tokens,
                                  int32_t* grow_to);
/* record_tokens: append n token ids (positions must already be reserved,
 * else PAGED_ERR_CAPACITY). */
int32_t paged_seq_commit_tokens(paged_alloc* a, int64_t seq_id, const int32_t* tokens,
                                int32_t n);
/* register_full_blocks_for_reuse: publish every full committed block that is
 * not yet published (stops at a null entry; a block whose key is already
 * published stays private and the chain continues through the published one). */
int32_t paged_seq_publish_full_blocks(paged_alloc* a, int64_t seq_id, uint64_t domain);
/* Sliding groups: replace by the null sentinel (0) every block lying wholly
 * before position committed_tokens - window, releasing it. */
int32_t paged_seq_drop_outside_window(paged_alloc* a, int64_t seq_id, int32_t window);
/* release_request: release every block (last entry first) and forget the sequence. */
int32_t paged_seq_release(paged_alloc* a, int64_t seq_id);
int32_t paged_seq_num_tokens(const paged_alloc* a, int64_t seq_id, int32_t* committed_tokens,
                             int32_t* table_blocks);

/* Host buffer out[batch][max_blocks], row b = table of seq_ids[b] padded with 0.
 * PAGED_ERR_CAPACITY (and *needed = widest table) if a table is wider. */
int32_t paged_alloc_block_tables(const paged_alloc* a, const int64_t* seq_ids, int32_t batch,
                                 int32_t max_blocks, int32_t* out, int32_t* needed);
/* Host buffer out[n] = slots of positions start_pos .. start_pos+n-1.
 * PAGED_ERR_CAPACITY for an unreserved position, PAGED_ERR_STATE for a
 * position in a dropped block; nothing is written when the call fails. */
int32_t paged_alloc_slot_mapping(const paged_alloc* a, int64_t seq_id, int32_t start_pos,
                                 int32_t n, int64_t* out);
int32_t paged_alloc_refcount(const paged_alloc* a, int32_t block_id, int32_t* refcount);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
