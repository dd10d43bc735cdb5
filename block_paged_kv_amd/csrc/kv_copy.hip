// Slot-mapped KV write and block-table gather (gfx950).
//
// mlx-node perf doc, paged-attention knobs table: the native paged K/V write
// scatters each new token's K and V rows into the slot its request owns, and
// the synchronous decode gather reads a row's pages (sliding groups from their
// first live block). Both are pure byte moves: each thread copies one 16-byte
// vector, so a token row of head_dim elements is moved by head_dim*esize/16
// consecutive lanes and every wave instruction touches contiguous memory on
// the source side.

#include <cmath>

#include "device.h"
#include "runtime.h"

namespace pagedkv {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void load16(const uint16_t* p, float* x) {
  const uint4 a = reinterpret_cast<const uint4*>(p)[0];
  const uint4 b = reinterpret_cast<const uint4*>(p)[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[2 * j] = bf16_lo(w[j]);
    x[2 * j + 1] = bf16_hi(w[j]);
  }
}

__device__ __forceinline__ void load16(const float* p, float* x) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 f = reinterpret_cast<const float4*>(p)[j];
    x[4 * j] = f.x;
    x[4 * j + 1] = f.y;
    x[4 * j + 2] = f.z;
    x[4 * j + 3] = f.w;
  }
}

// 16 values to 16 E4M3 codes (element 0 in the lowest byte).
__device__ __forceinline__ uint4 encode16(const float* x, float scale) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(x[4 * j + e] / scale, -448.f), 448.f);
    int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    packed = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], packed, true);
    w[j] = static_cast<uint32_t>(packed);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ __launch_bounds__(kThreads) void kv_write_kernel(
    uint4* __restrict__ k_pool, uint4* __restrict__ v_pool, const uint4* __restrict__ new_k,
    const uint4* __restrict__ new_v, const int64_t* __restrict__ slots, int64_t total_vecs,
    int32_t vecs_per_token, int32_t vecs_per_head, int32_t num_kv_heads, int32_t bs_log2,
    int64_t num_slots) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total_vecs;
       i += stride) {
    const int64_t t = i / vecs_per_token;
    const int32_t r = static_cast<int32_t>(i - t * vecs_per_token);
    // The data loads do not depend on the slot: issue all three together.
    const uint4 kv = new_k[i];
    const uint4 vv = new_v[i];
    const int64_t slot = slots[t];
    if ((slot >> bs_log2) <= 0 || slot >= num_slots) continue;  // padding, the null block, out of range
    const int32_t h = r / vecs_per_head;
    const int32_t v = r - h * vecs_per_head;
    const int64_t blk = slot >> bs_log2;
    const int64_t off = slot & ((1 << bs_log2) - 1);
    const int64_t dst = ((((blk * num_kv_heads + h) << bs_log2) + off) * vecs_per_head) + v;
    k_pool[dst] = kv;
    v_pool[dst] = vv;
  }
}

__global__ __launch_bounds__(kThreads) void kv_gather_kernel(
    uint4* __restrict__ out_k, uint4* __restrict__ out_v, const uint4* __restrict__ k_pool,
    const uint4* __restrict__ v_pool, const int32_t* __restrict__ block_tables, int32_t mb,
    const int32_t* __restrict__ seq_lens, const int64_t* __restrict__ out_offsets,
    int32_t max_seq_len, int32_t vecs_per_token, int32_t vecs_per_head, int32_t num_kv_heads,
    int32_t bs_log2, int32_t num_blocks, int32_t window) {
  const int b = blockIdx.y;
  const int n = min(seq_lens[b], max_seq_len);
  const int lo = window > 0 ? max(0, n - window) : 0;
  const int64_t total = static_cast<int64_t>(max(n - lo, 0)) * vecs_per_token;
  const int64_t base = out_offsets[b] * vecs_per_token;
  const int32_t* bt = block_tables + static_cast<int64_t>(b) * mb;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += stride) {
    const int64_t t = i / vecs_per_token;
    const int32_t r = static_cast<int32_t>(i - t * vecs_per_token);
    const int64_t p = lo + t;
    const int64_t lb = p >> bs_log2;
    if (lb >= mb) continue;
    const int32_t phys = bt[lb];
    if (phys <= 0 || phys >= num_blocks) continue;
    const int32_t h = r / vecs_per_head;
    const int32_t v = r - h * vecs_per_head;
    const int64_t src = ((((static_cast<int64_t>(phys) * num_kv_heads + h) << bs_log2) +
                          (p & ((1 << bs_log2) - 1))) * vecs_per_head) + v;
    out_k[base + i] = k_pool[src];
    out_v[base + i] = v_pool[src];
  }
}

// Quantizing write into FP8 pools: each thread produces 16 codes (one
// 16-byte store) from 16 source elements of one token row: x / scale in
// float32 (correctly rounded division), clamped to +-448, then the hardware
// E4M3 conversion (round to nearest even; it does not saturate by itself).
template <typename SRC>
__global__ __launch_bounds__(kThreads) void kv_write_fp8_kernel(
    uint4* __restrict__ k_pool, uint4* __restrict__ v_pool, const SRC* __restrict__ new_k,
    const SRC* __restrict__ new_v, const int64_t* __restrict__ slots, int64_t total_vecs,
    int32_t vecs_per_token, int32_t vecs_per_head, int32_t num_kv_heads, int32_t bs_log2,
    int64_t num_slots, float k_scale, float v_scale) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total_vecs;
       i += stride) {
    const int64_t t = i / vecs_per_token;
    const int32_t r = static_cast<int32_t>(i - t * vecs_per_token);
    float xk[16], xv[16];
    load16(new_k + i * 16, xk);
    load16(new_v + i * 16, xv);
    const int64_t slot = slots[t];
    if ((slot >> bs_log2) <= 0 || slot >= num_slots) continue;  // padding, the null block, out of range
    const int32_t h = r / vecs_per_head;
    const int32_t v = r - h * vecs_per_head;
    const int64_t blk = slot >> bs_log2;
    const int64_t off = slot & ((1 << bs_log2) - 1);
    const int64_t dst = ((((blk * num_kv_heads + h) << bs_log2) + off) * vecs_per_head) + v;
    k_pool[dst] = encode16(xk, k_scale);
    v_pool[dst] = encode16(xv, v_scale);
  }
}

int32_t check_common(int32_t head_dim, int32_t block_size, int32_t num_kv_heads, int32_t dtype) {
  if (esize_of(dtype) == 0) return fail(PAGED_ERR_DTYPE, "unknown dtype %d", dtype);
  if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
    return fail(PAGED_ERR_INVALID_ARG, "head_dim must be 64, 128, 256 or 512 (got %d)", head_dim);
  if (!pow2_in(block_size, 8, 64))
    return fail(PAGED_ERR_INVALID_ARG, "block_size must be a power of two in [8, 64] (got %d)",
                block_size);
  if (num_kv_heads < 1) return fail(PAGED_ERR_INVALID_ARG, "num_kv_heads must be positive");
  return PAGED_OK;
}

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

extern "C" int32_t paged_kv_write(void* k_pool, void* v_pool, const void* new_k, const void* new_v,
                                  const int64_t* slot_mapping, int32_t num_tokens,
                                  int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t dtype, void* stream) {
  if (int32_t rc = check_common(head_dim, block_size, num_kv_heads, dtype)) return rc;
  if (num_tokens < 0 || num_blocks < 1)
    return fail(PAGED_ERR_INVALID_ARG, "num_tokens >= 0 and num_blocks >= 1 required");
  if (num_tokens == 0) return ok();
  if (!k_pool || !v_pool || !new_k || !new_v || !slot_mapping)
    return fail(PAGED_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(new_k) || !aligned16(new_v) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
    return fail(PAGED_ERR_INVALID_ARG, "misaligned pointer");
  const int32_t vecs_per_head = head_dim * esize_of(dtype) / 16;
  const int32_t vecs_per_token = vecs_per_head * num_kv_heads;
  const int64_t total = static_cast<int64_t>(num_tokens) * vecs_per_token;
  const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 16384);
  hipStream_t s = static_cast<hipStream_t>(stream);
  LaunchTrace tr(PAGED_KERNEL_KV_WRITE, s);
  hipExtLaunchKernelGGL(kv_write_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s,
      tr.start(), tr.stop(), 0, static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), static_cast<const uint4*>(new_k),
      static_cast<const uint4*>(new_v), slot_mapping, total, vecs_per_token, vecs_per_head,
      num_kv_heads, ilog2(block_size), static_cast<int64_t>(num_blocks) * block_size);
  tr.finish();
  return check_launch("paged_kv_write");
}

extern "C" int32_t paged_kv_write_fp8(void* k_pool, void* v_pool, const void* new_k,
                                      const void* new_v, const int64_t* slot_mapping,
                                      int32_t num_tokens, int32_t num_blocks, int32_t block_size,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t src_dtype,
                                      float k_scale, float v_scale, void* stream) {
  if (src_dtype != PAGED_BF16 && src_dtype != PAGED_F32)
    return fail(PAGED_ERR_DTYPE, "source dtype must be bf16 or f32 (got %d)", src_dtype);
  if (int32_t rc = check_common(head_dim, block_size, num_kv_heads, PAGED_FP8_E4M3)) return rc;
  if (num_tokens < 0 || num_blocks < 1)
    return fail(PAGED_ERR_INVALID_ARG, "num_tokens >= 0 and num_blocks >= 1 required");
  if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(PAGED_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if (num_tokens == 0) return ok();
  if (!k_pool || !v_pool || !new_k || !new_v || !slot_mapping)
    return fail(PAGED_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(new_k) || !aligned16(new_v) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
    return fail(PAGED_ERR_INVALID_ARG, "misaligned pointer");
  const int32_t vecs_per_head = head_dim / 16;  // 16 codes per 16-byte vector
  const int32_t vecs_per_token = vecs_per_head * num_kv_heads;
  const int64_t total = static_cast<int64_t>(num_tokens) * vecs_per_token;
  const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 16384);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  LaunchTrace tr(PAGED_KERNEL_KV_WRITE, s);
  if (src_dtype == PAGED_BF16)
    hipExtLaunchKernelGGL(kv_write_fp8_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                          0, s, tr.start(), tr.stop(), 0, static_cast<uint4*>(k_pool),
                          static_cast<uint4*>(v_pool), static_cast<const uint16_t*>(new_k),
                          static_cast<const uint16_t*>(new_v), slot_mapping, total, vecs_per_token,
                          vecs_per_head, num_kv_heads, ilog2(block_size), num_slots, k_scale, v_scale);
  else
    hipExtLaunchKernelGGL(kv_write_fp8_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                          0, s, tr.start(), tr.stop(), 0, static_cast<uint4*>(k_pool),
                          static_cast<uint4*>(v_pool), static_cast<const float*>(new_k),
                          static_cast<const float*>(new_v), slot_mapping, total, vecs_per_token,
                          vecs_per_head, num_kv_heads, ilog2(block_size), num_slots, k_scale, v_scale);
  tr.finish();
  return check_launch("paged_kv_write_fp8");
}

extern "C" int32_t paged_kv_gather(void* out_k, void* out_v, const void* k_pool, const void* v_pool,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* seq_lens, const int64_t* out_offsets,
                                   int32_t batch, int32_t max_seq_len, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t sliding_window, int32_t dtype, void* stream) {
  if (int32_t rc = check_common(head_dim, block_size, num_kv_heads, dtype)) return rc;
  if (batch < 0 || max_seq_len < 0 || max_blocks_per_seq < 1 || num_blocks < 1 ||
      sliding_window < 0)
    return fail(PAGED_ERR_INVALID_ARG, "bad size argument");
  if (batch > 65535) return fail(PAGED_ERR_INVALID_ARG, "batch above 65535");
  if (batch == 0 || max_seq_len == 0) return ok();
  if (!out_k || !out_v || !k_pool || !v_pool || !block_tables || !seq_lens || !out_offsets)
    return fail(PAGED_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(out_k) || !aligned16(out_v) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PAGED_ERR_INVALID_ARG, "misaligned pointer");
  const int32_t vecs_per_head = head_dim * esize_of(dtype) / 16;
  const int32_t vecs_per_token = vecs_per_head * num_kv_heads;
  const int32_t span = sliding_window > 0 ? std::min(max_seq_len, sliding_window) : max_seq_len;
  const int64_t per_row = static_cast<int64_t>(span) * vecs_per_token;
  const int64_t gx = std::min<int64_t>((per_row + kThreads - 1) / kThreads, 4096);
  hipStream_t s = static_cast<hipStream_t>(stream);
  LaunchTrace tr(PAGED_KERNEL_KV_GATHER, s);
  hipExtLaunchKernelGGL(kv_gather_kernel, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(batch)),
                        dim3(kThreads), 0, s, tr.start(), tr.stop(), 0, static_cast<uint4*>(out_k), static_cast<uint4*>(out_v),
                             static_cast<const uint4*>(k_pool), static_cast<const uint4*>(v_pool),
                             block_tables, max_blocks_per_seq, seq_lens, out_offsets, max_seq_len,
                             vecs_per_token, vecs_per_head, num_kv_heads, ilog2(block_size),
                             num_blocks, sliding_window);
  tr.finish();
  return check_launch("paged_kv_gather");
}
