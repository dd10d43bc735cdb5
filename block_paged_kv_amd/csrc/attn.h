// Attention launchers shared between entry points (host side). Each checks its
// arguments, enqueues its kernels on `stream` and returns a PAGED_* status.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pagedkv {

// Split-K decode (partial + reduce) over pools of esz-byte elements: 4 float32,
// 2 bf16, 1 FP8 E4M3 codes (q and out bf16 then).
int32_t decode_impl(void* out, const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, float scale, float k_scale, float v_scale,
                    int32_t sliding_window, int32_t partition_tokens, int32_t max_seq_len,
                    void* workspace, size_t workspace_bytes, int esz, void* stream);

// Every argument check of decode_impl, with nothing enqueued.
int32_t decode_check(const void* out, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, float scale, float k_scale, float v_scale,
                     int32_t sliding_window, int32_t partition_tokens, int32_t max_seq_len,
                     const void* workspace, size_t workspace_bytes, int esz);

// Chunked prefill over pools of esz-byte elements (2 bf16, 1 FP8 codes); q and
// out bf16. cu_q_lens holds absolute offsets into q and out. workspace NULL: no key split; else
// the key split of the library rule, its partials in the workspace.
// beside_decode: the launch shares the device with decode work (mixed step),
// which changes only the order the query tiles are dispatched in.
int32_t prefill_impl(void* out, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* cu_q_lens, const int32_t* seq_lens, int32_t batch,
                     int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, float scale, float k_scale, float v_scale,
                     int32_t sliding_window, void* workspace, size_t workspace_bytes, int esz,
                     void* stream, bool beside_decode = false);

// Every argument check of prefill_impl, with nothing enqueued.
int32_t prefill_check(const void* out, const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* cu_q_lens, const int32_t* seq_lens, int32_t batch,
                      int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t num_blocks, float scale, float k_scale, float v_scale,
                      int32_t sliding_window);

}  // namespace pagedkv
