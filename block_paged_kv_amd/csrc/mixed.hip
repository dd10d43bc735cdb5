// One continuous-batching attention step: decode rows and prefill chunks of
// one batch in a single call (batching-perf-path doc, current state: chunked
// 2048-token prefill of joining requests interleaved with the running decode
// rows; paged-cache doc, hybrid coordinator paragraph for the sliding layers).
//
// What is computed is exactly paged_attn_prefill_chunk over the whole batch:
// a decode row is a chunk of one query at position n - 1. How (ours): the
// decode rows go through the split-K decode kernels on the caller's stream
// and the chunk rows through the prefill kernel on the library's side stream,
// so the bandwidth-bound decode and the matrix-core-bound prefill share the
// device instead of running one after the other; the caller's stream waits
// for both before anything enqueued after the call.

#include "attn.h"
#include "runtime.h"

using namespace pagedkv;

extern "C" int32_t paged_attn_mixed(void* out, const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* cu_q_lens, const int32_t* seq_lens, int32_t batch,
                                    int32_t num_decode_rows, int32_t total_q, int32_t max_q_len,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks, float scale,
                                    float k_scale, float v_scale, int32_t sliding_window,
                                    int32_t partition_tokens, int32_t max_seq_len, void* workspace,
                                    size_t workspace_bytes, int32_t kv_dtype, void* stream) {
  if (kv_dtype != PAGED_BF16 && kv_dtype != PAGED_FP8_E4M3)
    return fail(PAGED_ERR_DTYPE, "paged_attn_mixed takes bf16 or FP8 E4M3 pools (got dtype %d)", kv_dtype);
  const int esz = esize_of(kv_dtype);
  if (batch < 0 || num_decode_rows < 0 || num_decode_rows > batch || total_q < num_decode_rows ||
      max_blocks_per_seq < 1)
    return fail(PAGED_ERR_INVALID_ARG,
                "need 0 <= num_decode_rows <= batch, total_q >= num_decode_rows, max_blocks_per_seq >= 1");
  if (kv_dtype == PAGED_BF16 && (k_scale != 1.f || v_scale != 1.f))
    return fail(PAGED_ERR_INVALID_ARG, "k_scale and v_scale must be 1 for bf16 pools");
  const int32_t nd = num_decode_rows;
  const int32_t np = batch - nd;
  if (batch == 0) return ok();
  if (np == 0)
    return decode_impl(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, seq_lens, nd,
                       num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, k_scale,
                       v_scale, sliding_window, partition_tokens, max_seq_len, workspace,
                       workspace_bytes, esz, stream);
  if (nd == 0)
    return prefill_impl(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, cu_q_lens,
                        seq_lens, np, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim,
                        block_size, num_blocks, scale, k_scale, v_scale, sliding_window, nullptr, 0,
                        esz, stream);

  // Both parts: check everything either could reject before enqueuing anything.
  if (int32_t rc = prefill_check(out, q, k_pool, v_pool,
                                 block_tables + static_cast<size_t>(nd) * max_blocks_per_seq,
                                 max_blocks_per_seq, cu_q_lens + nd, seq_lens + nd, np, total_q - nd,
                                 max_q_len, num_q_heads, num_kv_heads, head_dim, block_size,
                                 num_blocks, scale, k_scale, v_scale, sliding_window))
    return rc;
  if (int32_t rc = decode_check(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, seq_lens, nd,
                                num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                                k_scale, v_scale, sliding_window, partition_tokens, max_seq_len,
                                workspace, workspace_bytes, esz))
    return rc;

  hipStream_t s = static_cast<hipStream_t>(stream);
  SideStream side(s);
  if (side.status() != PAGED_OK) return side.status();
  // Chunk rows first (the long kernel starts first), on the side stream: their
  // cu_q_lens entries are absolute offsets into q and out. The prefill keeps
  // its own workgroup shape; its query tiles go first-first (the default
  // order is last-first), which suited the decode beside it.
  int32_t rc = prefill_impl(out, q, k_pool, v_pool, block_tables + static_cast<size_t>(nd) * max_blocks_per_seq,
                            max_blocks_per_seq, cu_q_lens + nd, seq_lens + nd, np, total_q - nd,
                            max_q_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                            scale, k_scale, v_scale, sliding_window, /*workspace=*/nullptr, 0, esz,
                            side.get(), /*beside_decode=*/true);
  if (rc == PAGED_OK)
    rc = decode_impl(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, seq_lens, nd,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, k_scale,
                     v_scale, sliding_window, partition_tokens, max_seq_len, workspace,
                     workspace_bytes, esz, stream);
  const int32_t rj = side.join();
  return rc != PAGED_OK ? rc : rj;
}
