// Split-K GQA decode over a block-paged KV cache (gfx950).
//
// What is computed: for each row b and query head h, plain softmax attention
// of q[b][h] over the row's attended positions [lo, n), K/V read in place
// through the row's block table (mlx-node perf doc, paged-attention knobs
// table: batched multi-row paged decode, the decode gather reading sliding
// groups from their first live block; paged-cache doc, hybrid coordinator
// paragraph: null sentinel for expired sliding blocks).
//
// How (ours): the row's span, starting at the first live block, is cut into
// partitions of `part` positions (perf doc, attention-partitions paragraph:
// partitioned decode with a separate reducer; empty partitions add nothing).
// One workgroup of up to four 64-lane waves handles (row, KV head, group of
// GT query heads, partition). Memory mapping:
//   * a token row of K (head_dim elements, 128..512 bytes) is read by R = 16
//     (or 8) consecutive lanes with 16-byte loads, so one wave instruction
//     reads 64/R consecutive token rows = 1 KiB of one contiguous block slab;
//   * each iteration a lane issues 16 K loads and 16 V loads back to back
//     (32 KiB per wave in flight) before touching any of them;
//   * q.k is v_dot2_f32_bf16 (two bf16 products per instruction) followed by a
//     DPP sum over the R lanes of the row; the score is then known to every
//     lane of the row, so the online softmax runs per "token lane" with no
//     cross-row traffic, and P.V accumulates in fp32 in the lane that owns
//     those head_dim elements;
//   * the token lanes of a wave, then the waves of a workgroup (through LDS),
//     are merged once at the end. Partials are fp32 (max in log2 units, sum,
//     unnormalised accumulator); the reduce kernel combines them in partition
//     order, so results are deterministic and there are no atomics.

#include <cmath>

#include "device.h"
#include "runtime.h"

namespace pagedkv {
namespace {

constexpr int kMaxWaves = 4;

template <int ESZ, int D>
struct Geo {
  static constexpr int EPC = 16 / ESZ;                 // elements per 16-byte chunk
  static constexpr int CHUNKS = D / EPC;               // chunks per token row
  static constexpr int R = CHUNKS < 16 ? CHUNKS : 16;  // lanes sharing one token row
  static constexpr int CPL = CHUNKS / R;               // chunks per lane per token
  static constexpr int TPW = 64 / R;                   // token rows per wave load
  static constexpr int U = 16 / CPL;                   // token groups per iteration
  static constexpr int ITER = U * TPW;                 // tokens per wave iteration
  static constexpr int EPL = CPL * EPC;                // elements per lane per token
};

struct DecodeParams {
  void* out;       // direct mode (single partition): final output, else nullptr
  float* ws_acc;   // [B][Hq][max_parts][D] unnormalised accumulators
  float* ws_ml;    // [B][Hq][max_parts][2] (running max in log2 units, sum)
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* bt;
  const int32_t* seq_lens;
  int32_t batch, mb, hq, hkv, group, head_groups, bs_log2, nb, window, part, max_parts;
  float scale_log2;  // scale * log2(e)
};

template <int ESZ>
__device__ __forceinline__ float chunk_dot(const uint4& a, const uint4& b, float acc);

template <>
__device__ __forceinline__ float chunk_dot<2>(const uint4& a, const uint4& b, float acc) {
  acc = dot2_bf16(a.x, b.x, acc);
  acc = dot2_bf16(a.y, b.y, acc);
  acc = dot2_bf16(a.z, b.z, acc);
  return dot2_bf16(a.w, b.w, acc);
}

template <>
__device__ __forceinline__ float chunk_dot<4>(const uint4& a, const uint4& b, float acc) {
  acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
  acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
  acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
  return fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
}

// Unpack one 16-byte chunk to EPC floats.
template <int ESZ>
__device__ __forceinline__ void chunk_unpack(const uint4& c, float* f) {
  if constexpr (ESZ == 2) {
    f[0] = bf16_lo(c.x); f[1] = bf16_hi(c.x);
    f[2] = bf16_lo(c.y); f[3] = bf16_hi(c.y);
    f[4] = bf16_lo(c.z); f[5] = bf16_hi(c.z);
    f[6] = bf16_lo(c.w); f[7] = bf16_hi(c.w);
  } else {
    f[0] = __uint_as_float(c.x); f[1] = __uint_as_float(c.y);
    f[2] = __uint_as_float(c.z); f[3] = __uint_as_float(c.w);
  }
}

template <int ESZ>
__device__ __forceinline__ void store_out(void* out, size_t idx, float v) {
  if constexpr (ESZ == 2)
    static_cast<uint16_t*>(out)[idx] = static_cast<uint16_t>(f32_to_bf16_bits(v));
  else
    static_cast<float*>(out)[idx] = v;
}

// Cross-wave merge through LDS and the partition's store, shared by both
// partial kernels. On entry m[g], l[g] are the wave's running max (log2 units)
// and sum for query head h0+g (uniform across the wave) and acc[g][.] holds the
// wave's unnormalised accumulator for the head_dim elements (j*R + sub)*EPC + e
// this lane owns, identical in every token lane of the wave.
template <int ESZ, int D, int GT, int R, int CPL>
__device__ __forceinline__ void write_partition(const DecodeParams& a, int p, int b, int h0,
                                                const float (&m)[GT], const float (&l)[GT],
                                                const float (&acc)[GT][CPL * (16 / ESZ)],
                                                float (*sm_acc)[GT][D], float (*sm_m)[GT],
                                                float (*sm_l)[GT]) {
  constexpr int EPC = 16 / ESZ;
  constexpr float kNegInf = -INFINITY;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int sub = lane % R;
  const int tl = lane / R;
  if (tl == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int e = 0; e < EPC; ++e) sm_acc[wave][g][(j * R + sub) * EPC + e] = acc[g][j * EPC + e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      sm_m[wave][g] = m[g];
      sm_l[wave][g] = l[g];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < GT * D; i += blockDim.x) {
    const int g = i / D;
    const int d = i - g * D;
    float M = kNegInf;
    for (int w = 0; w < nw; ++w) M = fmaxf(M, sm_m[w][g]);
    float L = 0.f, A = 0.f;
    for (int w = 0; w < nw; ++w) {
      const float mw = sm_m[w][g];
      const float f = mw == kNegInf ? 0.f : fast_exp2(mw - M);
      L += sm_l[w][g] * f;
      A += sm_acc[w][g][d] * f;
    }
    const size_t bh = static_cast<size_t>(b) * a.hq + h0 + g;
    if (a.out) {
      store_out<ESZ>(a.out, bh * D + d, L > 0.f ? A / L : 0.f);
    } else {
      const size_t slot = bh * a.max_parts + p;
      a.ws_acc[slot * D + d] = A;
      if (d == 0) {
        a.ws_ml[slot * 2] = M;
        a.ws_ml[slot * 2 + 1] = L;
      }
    }
  }
}

template <int ESZ, int D, int GT>
__global__ __launch_bounds__(64 * kMaxWaves) void decode_partial_kernel(DecodeParams a) {
  using Gm = Geo<ESZ, D>;
  constexpr int R = Gm::R, CPL = Gm::CPL, TPW = Gm::TPW, U = Gm::U, ITER = Gm::ITER;
  constexpr int EPC = Gm::EPC, EPL = Gm::EPL;
  constexpr float kNegInf = -INFINITY;

  __shared__ float sm_acc[kMaxWaves][GT][D];
  __shared__ float sm_m[kMaxWaves][GT];
  __shared__ float sm_l[kMaxWaves][GT];

  const int p = blockIdx.x;
  const int hg = blockIdx.y;
  const int b = blockIdx.z;
  const int kvh = hg / a.head_groups;
  const int h0 = kvh * a.group + (hg - kvh * a.head_groups) * GT;
  const int n = a.seq_lens[b];
  const int lo = a.window > 0 ? max(0, n - a.window) : 0;
  const int s0 = (lo >> a.bs_log2) << a.bs_log2;
  const int ps = s0 + p * a.part;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;

  if (ps >= n) {
    // Only an empty row (n == 0) reaches this with p == 0: its output is zero.
    if (a.out && p == 0)
      for (int i = threadIdx.x; i < GT * D; i += blockDim.x)
        store_out<ESZ>(a.out, (static_cast<size_t>(b) * a.hq + h0) * D + i, 0.f);
    return;
  }
  const int t_begin = max(ps, lo);
  const int t_end = min(ps + a.part, n);
  const int sub = lane % R;
  const int tl = lane / R;
  const int bs_mask = (1 << a.bs_log2) - 1;

  uint4 qv[GT][CPL];
  {
    const char* qb = static_cast<const char*>(a.q) + (static_cast<size_t>(b) * a.hq + h0) * D * ESZ;
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        qv[g][j] = *reinterpret_cast<const uint4*>(qb + g * D * ESZ + (j * R + sub) * 16);
  }

  float m[GT], l[GT], acc[GT][EPL];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  const int32_t* bt = a.bt + static_cast<size_t>(b) * a.mb;
  const char* kpool = static_cast<const char*>(a.k_pool);
  const char* vpool = static_cast<const char*>(a.v_pool);

  // Block-table entries of one iteration: lane l holds the entry of the l-th
  // block the iteration touches (one load per wave instead of one dependent
  // load per token group). The next iteration's entries are prefetched while
  // this iteration's K/V loads are in flight.
  const int it_blocks = ITER > (1 << a.bs_log2) ? (ITER >> a.bs_log2) : 1;
  auto load_table = [&](int it) -> int {
    const int lb = (it >> a.bs_log2) + lane;
    return (it < t_end && lane < it_blocks && lb < a.mb && (lb << a.bs_log2) < t_end) ? bt[lb] : 0;
  };
  int tbl = load_table(ps + wave * ITER);

  for (int it = ps + wave * ITER; it < t_end; it += nw * ITER) {
    uint4 kr[U][CPL], vr[U][CPL];
    bool valid[U];
    const int blk0 = it >> a.bs_log2;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tg = it + u * TPW;  // first token of this group (wave-uniform)
      const int phys = __builtin_amdgcn_readlane(tbl, (tg >> a.bs_log2) - blk0);
      const int t = tg + tl;
      valid[u] = t >= t_begin && t < t_end && phys > 0 && phys < a.nb;
      const size_t row = ((static_cast<size_t>(phys) * a.hkv + kvh) << a.bs_log2) + (t & bs_mask);
      const char* kp = kpool + row * (D * ESZ) + sub * 16;
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        kr[u][j] = valid[u] ? *reinterpret_cast<const uint4*>(kp + j * R * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tg = it + u * TPW;
      const int phys = __builtin_amdgcn_readlane(tbl, (tg >> a.bs_log2) - blk0);
      const int t = tg + tl;
      const size_t row = ((static_cast<size_t>(phys) * a.hkv + kvh) << a.bs_log2) + (t & bs_mask);
      const char* vp = vpool + row * (D * ESZ) + sub * 16;
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        vr[u][j] = valid[u] ? *reinterpret_cast<const uint4*>(vp + j * R * 16) : make_uint4(0, 0, 0, 0);
    }
    tbl = load_table(it + nw * ITER);

    // Scores in log2 units; every lane of a token row ends with the same value.
    float s[U][GT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) d = chunk_dot<ESZ>(qv[g][j], kr[u][j], d);
        d = group_sum<R>(d);
        s[u][g] = valid[u] ? d * a.scale_log2 : kNegInf;
      }

    // Online softmax per token lane: new max, rescale, probabilities.
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u][g]);
      const float mref = mx == kNegInf ? 0.f : mx;
      const float alpha = fast_exp2(m[g] - mref);
      float ls = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float pr = fast_exp2(s[u][g] - mref);
        s[u][g] = pr;
        ls += pr;
      }
      l[g] = l[g] * alpha + ls;
      m[g] = mx;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
    }

    // P.V in fp32; invalid tokens have p = 0 and zeroed V.
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        float vf[EPC];
        chunk_unpack<ESZ>(vr[u][j], vf);
#pragma unroll
        for (int g = 0; g < GT; ++g)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[g][j * EPC + e] = fmaf(s[u][g], vf[e], acc[g][j * EPC + e]);
      }
  }

  // Merge the token lanes of this wave (lanes that differ by multiples of R).
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    float M = m[g];
#pragma unroll
    for (int off = R; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float f = m[g] == kNegInf ? 0.f : fast_exp2(m[g] - M);
    float lw = l[g] * f;
#pragma unroll
    for (int off = R; off < 64; off <<= 1) lw += __shfl_xor(lw, off);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = acc[g][e] * f;
#pragma unroll
      for (int off = R; off < 64; off <<= 1) x += __shfl_xor(x, off);
      acc[g][e] = x;
    }
    m[g] = M;
    l[g] = lw;
  }

  write_partition<ESZ, D, GT, R, CPL>(a, p, b, h0, m, l, acc, sm_acc, sm_m, sm_l);
}

// ---------------------------------------------------------------------------
// bf16 decode with q.K on the matrix cores.
//
// Per 16-token K tile, S = Q K^T is one v_mfma_f32_16x16x32_bf16 per 32
// head_dim elements: the A operand holds the (up to 8) query heads of the
// group as rows (zero-padded to 16), the B operand the tile's 16 keys. K is
// loaded in exactly that operand layout -- lane l reads 16 bytes of token
// l%16 -- so the token a lane loads is also the score column it receives, and
// validity masks need no shuffle. Lane l then holds the scores of heads
// 4*(l/16)+i, i < 4, for token l%16 of each tile: the row max is a 16-lane DPP
// reduction, and probabilities go through a small per-wave LDS buffer to the
// P.V layout. P.V stays on VALU: V is read 16 bytes per lane with R = D/8 lanes
// per token row (coalesced; each lane owns 8 head_dim elements, so the fp32
// accumulators take GT*8 registers), and two tokens at a time are combined by
// v_dot2_f32_bf16 on bf16 (p_a, p_b) and (v_a, v_b) pairs built with v_perm.
// Probabilities are rounded to bf16 for that product only; max, sum and the
// accumulators stay fp32.
template <int D, int GT>
struct MfmaGeo {
  static constexpr int KS = D / 32;                        // MFMA k-steps per K tile
  static constexpr int KT = D == 64 ? 8 : D == 128 ? 4 : 2;  // K tiles per iteration
  static constexpr int NTOK = 16 * KT;                     // tokens per wave iteration
  static constexpr int R = D / 8;                          // V: lanes per token row (8..32)
  static constexpr int CPL = (D / 8) / R;                  // V: 16-byte chunks per lane per token
  static constexpr int TPW = 64 / R;                       // V: token rows per wave load
  static constexpr int U = NTOK / TPW;                     // V: token groups per iteration (even)
  static constexpr int EPL = CPL * 8;                      // V: head_dim elements per lane
  static constexpr int GTP = GT <= 4 ? 4 : 8;              // heads per token in the p buffer
};

template <int R>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (R >= 2) x = fmaxf(x, dpp_mov<0xB1>(x));
  if constexpr (R >= 4) x = fmaxf(x, dpp_mov<0x4E>(x));
  if constexpr (R >= 8) x = fmaxf(x, dpp_mov<0x141>(x));
  if constexpr (R >= 16) x = fmaxf(x, dpp_mov<0x140>(x));
  return x;
}

typedef __bf16 bf16x8v_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx4_t mfma_16x16x32(const uint4& a, const uint4& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v_t, a),
                                                 __builtin_bit_cast(bf16x8v_t, b), c, 0, 0, 0);
}

template <int D, int GT>
__global__ __launch_bounds__(64 * kMaxWaves, 2) void decode_partial_mfma_kernel(DecodeParams a) {
  using Gm = MfmaGeo<D, GT>;
  constexpr int KS = Gm::KS, KT = Gm::KT, NTOK = Gm::NTOK, R = Gm::R, CPL = Gm::CPL;
  constexpr int TPW = Gm::TPW, U = Gm::U, EPL = Gm::EPL, GTP = Gm::GTP;
  constexpr float kNegInf = -INFINITY;

  __shared__ float sm_acc[kMaxWaves][GT][D];
  __shared__ float sm_m[kMaxWaves][GT];
  __shared__ float sm_l[kMaxWaves][GT];
  __shared__ __attribute__((aligned(16))) float sm_p[kMaxWaves][NTOK * GTP];

  const int p = blockIdx.x;
  const int hg = blockIdx.y;
  const int b = blockIdx.z;
  const int kvh = hg / a.head_groups;
  const int h0 = kvh * a.group + (hg - kvh * a.head_groups) * GT;
  const int n = a.seq_lens[b];
  const int lo = a.window > 0 ? max(0, n - a.window) : 0;
  const int s0 = (lo >> a.bs_log2) << a.bs_log2;
  const int ps = s0 + p * a.part;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;

  if (ps >= n) {
    // Only an empty row (n == 0) reaches this with p == 0: its output is zero.
    if (a.out && p == 0)
      for (int i = threadIdx.x; i < GT * D; i += blockDim.x)
        store_out<2>(a.out, (static_cast<size_t>(b) * a.hq + h0) * D + i, 0.f);
    return;
  }
  const int t_begin = max(ps, lo);
  const int t_end = min(ps + a.part, n);
  const int lq = lane & 15;  // K: token within a tile; S: score column
  const int lg = lane >> 4;  // K: 16-byte chunk group; S: head group (heads 4*lg + i)
  const int sub = lane % R;  // V: chunk within the token row
  const int tl = lane / R;   // V: token within a group
  const int bs_log2 = a.bs_log2;
  const int bs_mask = (1 << bs_log2) - 1;

  // A operand: head row lq (zero beyond GT), elements 8*(lg + 4j) .. +8 of step j.
  uint4 qa[KS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<size_t>(b) * a.hq + h0 + (lq < GT ? lq : 0)) * D;
#pragma unroll
    for (int j = 0; j < KS; ++j)
      qa[j] = lq < GT ? *reinterpret_cast<const uint4*>(qrow + 8 * (lg + 4 * j)) : make_uint4(0, 0, 0, 0);
  }

  float mrun[4], lrun[4];  // S layout: heads 4*lg + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mrun[i] = kNegInf;
    lrun[i] = 0.f;
  }
  float acc[GT][EPL];      // V layout: head_dim elements (j*R + sub)*8 + e
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;

  const int32_t* bt = a.bt + static_cast<size_t>(b) * a.mb;
  const char* kpool = static_cast<const char*>(a.k_pool);
  const char* vpool = static_cast<const char*>(a.v_pool);
  const float c = a.scale_log2;
  float* pbuf = sm_p[wave];

  // Table entries of one iteration (lane l: l-th block), prefetched one ahead.
  const int it_blocks = NTOK > (1 << bs_log2) ? (NTOK >> bs_log2) : 1;
  auto load_table = [&](int it) -> int {
    const int lb = (it >> bs_log2) + lane;
    return (it < t_end && lane < it_blocks && lb < a.mb && (lb << bs_log2) < t_end) ? bt[lb] : 0;
  };
  int tbl = load_table(ps + wave * NTOK);

  for (int it = ps + wave * NTOK; it < t_end; it += nw * NTOK) {
    const int blk0 = it >> bs_log2;
    uint4 kb[KT][KS];
    bool kval[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const int tok = it + 16 * t + lq;
      const int phys = __shfl(tbl, (tok >> bs_log2) - blk0);
      kval[t] = tok >= t_begin && tok < t_end && phys > 0 && phys < a.nb;
      const char* src = kpool + ((((static_cast<size_t>(phys) * a.hkv + kvh) << bs_log2) + (tok & bs_mask)) * D +
                                 8 * lg) * 2;
      if (kval[t]) {
#pragma unroll
        for (int j = 0; j < KS; ++j) kb[t][j] = *reinterpret_cast<const uint4*>(src + 64 * j);
      } else {
#pragma unroll
        for (int j = 0; j < KS; ++j) kb[t][j] = make_uint4(0, 0, 0, 0);
      }
    }
    uint4 vr[U][CPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tg = it + TPW * u;
      const int phys = __builtin_amdgcn_readlane(tbl, (tg >> bs_log2) - blk0);
      const int tok = tg + tl;
      const bool ok = tok >= t_begin && tok < t_end && phys > 0 && phys < a.nb;
      const char* src = vpool + ((((static_cast<size_t>(phys) * a.hkv + kvh) << bs_log2) + (tok & bs_mask)) * D) * 2 +
                        16 * sub;
      if (ok) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) vr[u][j] = *reinterpret_cast<const uint4*>(src + 16 * R * j);
      } else {
#pragma unroll
        for (int j = 0; j < CPL; ++j) vr[u][j] = make_uint4(0, 0, 0, 0);
      }
    }
    tbl = load_table(it + nw * NTOK);

    // ---- scores on MFMA: lane holds S[4*lg + i][16t + lq] ---------------------
    floatx4_t sacc[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      sacc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KS; ++j) sacc[t] = mfma_16x16x32(qa[j], kb[t][j], sacc[t]);
    }

    // ---- online softmax over this iteration's tokens ----------------------------
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const float v = kval[t] ? sacc[t][i] * c : kNegInf;
        sacc[t][i] = v;
        mx = fmaxf(mx, v);
      }
      mx = group_max<16>(mx);
      const float mnew = fmaxf(mrun[i], mx);
      const float mref = mnew == kNegInf ? 0.f : mnew;
      alpha[i] = fast_exp2(mrun[i] - mref);
      mrun[i] = mnew;
      float ls = 0.f;
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const float pr = fast_exp2(sacc[t][i] - mref);
        sacc[t][i] = pr;
        ls += pr;
      }
      lrun[i] = lrun[i] * alpha[i] + ls;
    }
    if (lg < GTP / 4) {
#pragma unroll
      for (int t = 0; t < KT; ++t)
        *reinterpret_cast<float4*>(&pbuf[(16 * t + lq) * GTP + 4 * lg]) =
            make_float4(sacc[t][0], sacc[t][1], sacc[t][2], sacc[t][3]);
    }
    // Rescale the accumulators of heads whose running max moved.
    float al[GT];
    bool moved = false;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      al[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[g & 3]), 16 * (g >> 2)));
      moved |= al[g] != 1.f;
    }
    if (moved) {
#pragma unroll
      for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= al[g];
    }
    __builtin_amdgcn_wave_barrier();

    // ---- P.V on VALU: tokens TPW*u + tl and TPW*(u+1) + tl per dot2 ----------
#pragma unroll
    for (int u = 0; u < U; u += 2) {
      const float* pa = &pbuf[(TPW * u + tl) * GTP];
      const float* pb = &pbuf[(TPW * (u + 1) + tl) * GTP];
      uint32_t pp[GT];
#pragma unroll
      for (int g = 0; g < GT; ++g) pp[g] = pack_bf16x2(pa[g], pb[g]);
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const uint32_t* va = reinterpret_cast<const uint32_t*>(&vr[u][j]);
        const uint32_t* vb = reinterpret_cast<const uint32_t*>(&vr[u + 1][j]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo2 = __builtin_amdgcn_perm(vb[w], va[w], 0x05040100u);
          const uint32_t hi2 = __builtin_amdgcn_perm(vb[w], va[w], 0x07060302u);
#pragma unroll
          for (int g = 0; g < GT; ++g) {
            acc[g][j * 8 + 2 * w] = dot2_bf16(pp[g], lo2, acc[g][j * 8 + 2 * w]);
            acc[g][j * 8 + 2 * w + 1] = dot2_bf16(pp[g], hi2, acc[g][j * 8 + 2 * w + 1]);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // Wave totals: sum over the 16 score lanes (l) and over the token lanes (acc).
  float m[GT], l[GT];
#pragma unroll
  for (int i = 0; i < 4; ++i) lrun[i] = group_sum<16>(lrun[i]);
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mrun[g & 3]), 16 * (g >> 2)));
    l[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lrun[g & 3]), 16 * (g >> 2)));
  }
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = acc[g][e];
#pragma unroll
      for (int off = R; off < 64; off <<= 1) x += __shfl_xor(x, off);
      acc[g][e] = x;
    }
  write_partition<2, D, GT, R, CPL>(a, p, b, h0, m, l, acc, sm_acc, sm_m, sm_l);
}


// One wave per (row, query head): combine that pair's partitions in order.
// Lane p reads partition p's (max, sum) so all of them arrive in one round
// trip; the accumulators are then summed in partition order with the loads of
// eight partitions in flight at a time.
template <int ESZ, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeParams a) {
  constexpr float kNegInf = -INFINITY;
  constexpr int PER_LANE = D / 64;
  __shared__ float sm_w[4][64];
  const int wave = threadIdx.x >> 6;
  const int pair = blockIdx.x * 4 + wave;
  if (pair >= a.batch * a.hq) return;
  const int lane = threadIdx.x & 63;
  const int b = pair / a.hq;
  const int n = a.seq_lens[b];
  const int lo = a.window > 0 ? max(0, n - a.window) : 0;
  const int s0 = (lo >> a.bs_log2) << a.bs_log2;
  const int np = n > s0 ? min((n - s0 + a.part - 1) / a.part, a.max_parts) : 0;
  const float* ml = a.ws_ml + static_cast<size_t>(pair) * a.max_parts * 2;
  const float* acc = a.ws_acc + static_cast<size_t>(pair) * a.max_parts * D;
  float o[PER_LANE];
#pragma unroll
  for (int k = 0; k < PER_LANE; ++k) o[k] = 0.f;
  float L = 0.f;
  for (int p0 = 0; p0 < np; p0 += 64) {
    // (max, sum) of partitions p0 + lane; the running max M covers all chunks.
    const int p = p0 + lane;
    const float mp = p < np ? ml[2 * p] : kNegInf;
    const float lp = p < np ? ml[2 * p + 1] : 0.f;
    float M = mp;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    // Chunks beyond the first (more than 64 partitions) rescale what came before.
    if (p0 > 0) {
      const float prevM = sm_w[wave][0];
      const float newM = fmaxf(prevM, M);
      const float f = prevM == kNegInf ? 0.f : fast_exp2(prevM - newM);
      L *= f;
#pragma unroll
      for (int k = 0; k < PER_LANE; ++k) o[k] *= f;
      M = newM;
    }
    const float w = mp == kNegInf ? 0.f : fast_exp2(mp - M);
    float lw = lp * w;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lw += __shfl_xor(lw, off);
    L += lw;
    __builtin_amdgcn_wave_barrier();
    sm_w[wave][lane] = w;
    __builtin_amdgcn_wave_barrier();
    const int cnt = min(64, np - p0);
    int q = 0;
    for (; q + 8 <= cnt; q += 8) {
      float x[8][PER_LANE];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int k = 0; k < PER_LANE; ++k)
          x[i][k] = acc[static_cast<size_t>(p0 + q + i) * D + lane + 64 * k];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int k = 0; k < PER_LANE; ++k) o[k] = fmaf(x[i][k], sm_w[wave][q + i], o[k]);
    }
    for (; q < cnt; ++q)
#pragma unroll
      for (int k = 0; k < PER_LANE; ++k)
        o[k] = fmaf(acc[static_cast<size_t>(p0 + q) * D + lane + 64 * k], sm_w[wave][q], o[k]);
    __builtin_amdgcn_wave_barrier();
    if (lane == 0) sm_w[wave][0] = M;
    __builtin_amdgcn_wave_barrier();
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int k = 0; k < PER_LANE; ++k)
    store_out<ESZ>(a.out, static_cast<size_t>(pair) * D + lane + 64 * k, o[k] * inv);
}

// Tokens one wave processes per iteration, for the kernel a call dispatches to.
int iter_tokens_rt(int esz, int d, int gt) {
  if (esz == 2) {
    switch (d) {
      case 64: return MfmaGeo<64, 1>::NTOK;
      case 128: return MfmaGeo<128, 1>::NTOK;
      default: return MfmaGeo<256, 1>::NTOK;
    }
  }
  return d == 64 ? Geo<4, 64>::ITER : d == 128 ? Geo<4, 128>::ITER : Geo<4, 256>::ITER;
}

// Query heads one workgroup handles: the largest supported size dividing the
// group (bf16 kernel: 8, 6, 4, 3, 2, 1; fp32 kernel: 4, 2, 1).
int head_group_size(int group, int esz) {
  static const int kBf16[] = {8, 6, 4, 3, 2, 1};
  static const int kF32[] = {4, 2, 1};
  if (esz == 2) {
    for (int g : kBf16)
      if (group % g == 0) return g;
  } else {
    for (int g : kF32)
      if (group % g == 0) return g;
  }
  return 1;
}

int32_t span_tokens(int32_t max_seq_len, int32_t window, int32_t block_size) {
  return window > 0 ? std::min(max_seq_len, window + block_size - 1) : max_seq_len;
}

struct Plan {
  int32_t part, max_parts, nw, gt;
  bool direct;
  size_t ws_bytes;
};

int32_t make_plan(int32_t batch, int32_t hq, int32_t hkv, int32_t head_dim, int32_t block_size,
                  int32_t max_seq_len, int32_t window, int32_t partition_tokens, int esz, Plan* pl) {
  if (batch < 0 || hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(PAGED_ERR_INVALID_ARG, "need num_q_heads a positive multiple of num_kv_heads");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(PAGED_ERR_INVALID_ARG, "head_dim must be 64, 128 or 256 (got %d)", head_dim);
  if (!pow2_in(block_size, 8, 64))
    return fail(PAGED_ERR_INVALID_ARG, "block_size must be a power of two in [8, 64]");
  if (max_seq_len < 0 || window < 0) return fail(PAGED_ERR_INVALID_ARG, "negative length");
  const int group = hq / hkv;
  pl->gt = head_group_size(group, esz);
  const int32_t span = span_tokens(max_seq_len, window, block_size);
  int32_t part = partition_tokens;
  if (part == 0) {
    const int cus = device_cu_count();
    if (cus <= 0) return fail(PAGED_ERR_HIP, "cannot query the device compute-unit count");
    const int64_t wgs_per_part = static_cast<int64_t>(batch) * hkv * (group / pl->gt);
    part = 64;
    for (int32_t c = 1024; c >= 64; c >>= 1) {
      if (wgs_per_part * ((span + c - 1) / c) >= 4LL * cus) {
        part = c;
        break;
      }
    }
    part = std::max(part, block_size);
  }
  if (part < 16 || part > 65536 || part % block_size != 0)
    return fail(PAGED_ERR_INVALID_ARG,
                "partition_tokens must be a multiple of block_size in [16, 65536] (got %d)", part);
  pl->part = part;
  pl->max_parts = std::max(1, (span + part - 1) / part);
  pl->direct = pl->max_parts == 1;
  // Waves per workgroup: long-lived waves stream best, so each wave gets at
  // least 4 iterations of its partition (1..4 waves). The choice depends on
  // the partition size only, so a larger max_seq_len (extra, empty
  // partitions) never changes how a row's partials are merged.
  const int iter = iter_tokens_rt(esz, head_dim, pl->gt);
  const int iters = (part + iter - 1) / iter;
  pl->nw = std::min(kMaxWaves, std::max(1, iters / 4));
  pl->ws_bytes = pl->direct ? 0
                            : static_cast<size_t>(batch) * hq * pl->max_parts *
                                  (static_cast<size_t>(head_dim) + 2) * sizeof(float);
  return PAGED_OK;
}

template <int D>
void launch_partial_f32(const DecodeParams& prm, int gt, dim3 grid, dim3 block, hipStream_t s,
                        const LaunchTrace& tr) {
  switch (gt) {
    case 4: hipExtLaunchKernelGGL(decode_partial_kernel<4, D, 4>, grid, block, 0, s, tr.start(), tr.stop(), 0, prm); break;
    case 2: hipExtLaunchKernelGGL(decode_partial_kernel<4, D, 2>, grid, block, 0, s, tr.start(), tr.stop(), 0, prm); break;
    default: hipExtLaunchKernelGGL(decode_partial_kernel<4, D, 1>, grid, block, 0, s, tr.start(), tr.stop(), 0, prm); break;
  }
}

template <int D>
void launch_partial_bf16(const DecodeParams& prm, int gt, dim3 grid, dim3 block, hipStream_t s,
                         const LaunchTrace& tr) {
  switch (gt) {
    case 8: hipExtLaunchKernelGGL(decode_partial_mfma_kernel<D, 8>, grid, block, 0, s, tr.start(), tr.stop(), 0, prm); break;
    case 6: hipExtLaunchKernelGGL(decode_partial_mfma_kernel<D, 6>, grid, block, 0, s, tr.start(), tr.stop(), 0, prm); break;
    case 4: hipExtLaunchKernelGGL(decode_partial_mfma_kernel<D, 4>, grid, block, 0, s, tr.start(), tr.stop(), 0, prm); break;
    case 3: hipExtLaunchKernelGGL(decode_partial_mfma_kernel<D, 3>, grid, block, 0, s, tr.start(), tr.stop(), 0, prm); break;
    case 2: hipExtLaunchKernelGGL(decode_partial_mfma_kernel<D, 2>, grid, block, 0, s, tr.start(), tr.stop(), 0, prm); break;
    default: hipExtLaunchKernelGGL(decode_partial_mfma_kernel<D, 1>, grid, block, 0, s, tr.start(), tr.stop(), 0, prm); break;
  }
}

void launch_partial_any(const DecodeParams& prm, int esz, int d, int gt, dim3 grid, dim3 block,
                        hipStream_t s, const LaunchTrace& tr) {
  if (esz == 2) {
    if (d == 64) launch_partial_bf16<64>(prm, gt, grid, block, s, tr);
    else if (d == 128) launch_partial_bf16<128>(prm, gt, grid, block, s, tr);
    else launch_partial_bf16<256>(prm, gt, grid, block, s, tr);
  } else {
    if (d == 64) launch_partial_f32<64>(prm, gt, grid, block, s, tr);
    else if (d == 128) launch_partial_f32<128>(prm, gt, grid, block, s, tr);
    else launch_partial_f32<256>(prm, gt, grid, block, s, tr);
  }
}

template <int ESZ>
void launch_reduce_d(const DecodeParams& prm, int d, dim3 grid, hipStream_t s, const LaunchTrace& tr) {
  if (d == 64)
    hipExtLaunchKernelGGL(decode_reduce_kernel<ESZ, 64>, grid, dim3(256), 0, s, tr.start(), tr.stop(), 0, prm);
  else if (d == 128)
    hipExtLaunchKernelGGL(decode_reduce_kernel<ESZ, 128>, grid, dim3(256), 0, s, tr.start(), tr.stop(), 0, prm);
  else
    hipExtLaunchKernelGGL(decode_reduce_kernel<ESZ, 256>, grid, dim3(256), 0, s, tr.start(), tr.stop(), 0, prm);
}

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

extern "C" int32_t paged_attn_decode_partition_tokens(int32_t batch, int32_t num_q_heads,
                                                      int32_t num_kv_heads, int32_t block_size,
                                                      int32_t max_seq_len, int32_t sliding_window,
                                                      int32_t* partition_tokens) {
  if (!partition_tokens) return fail(PAGED_ERR_INVALID_ARG, "NULL argument");
  Plan pl;
  if (int32_t rc = make_plan(batch, num_q_heads, num_kv_heads, 128, block_size, max_seq_len,
                             sliding_window, 0, 2, &pl))
    return rc;
  *partition_tokens = pl.part;
  return ok();
}

extern "C" int32_t paged_attn_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                                     int32_t num_kv_heads, int32_t head_dim,
                                                     int32_t block_size, int32_t max_seq_len,
                                                     int32_t sliding_window,
                                                     int32_t partition_tokens, size_t* bytes) {
  if (!bytes) return fail(PAGED_ERR_INVALID_ARG, "NULL argument");
  Plan pl;
  if (int32_t rc = make_plan(batch, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len,
                             sliding_window, partition_tokens, 2, &pl))
    return rc;
  *bytes = pl.ws_bytes;
  return ok();
}

extern "C" int32_t paged_attn_decode(void* out, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                     int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     float scale, int32_t sliding_window,
                                     int32_t partition_tokens, int32_t max_seq_len,
                                     void* workspace, size_t workspace_bytes, int32_t dtype,
                                     void* stream) {
  const int esz = esize_of(dtype);
  if (esz == 0) return fail(PAGED_ERR_DTYPE, "unknown dtype %d", dtype);
  Plan pl;
  if (int32_t rc = make_plan(batch, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len,
                             sliding_window, partition_tokens, esz, &pl))
    return rc;
  if (max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(PAGED_ERR_INVALID_ARG, "max_blocks_per_seq and num_blocks must be positive");
  if (!std::isfinite(scale)) return fail(PAGED_ERR_INVALID_ARG, "scale must be finite");
  if (batch > 65535 || num_q_heads > 65535)
    return fail(PAGED_ERR_INVALID_ARG, "batch and num_q_heads must be at most 65535");
  if (batch == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !seq_lens)
    return fail(PAGED_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PAGED_ERR_INVALID_ARG, "misaligned pointer");
  if (!pl.direct) {
    if (!workspace || !aligned16(workspace))
      return fail(PAGED_ERR_INVALID_ARG, "workspace is NULL or misaligned");
    if (workspace_bytes < pl.ws_bytes)
      return fail(PAGED_ERR_CAPACITY, "workspace needs %zu bytes, got %zu", pl.ws_bytes,
                  workspace_bytes);
  }
  DecodeParams prm{};
  prm.out = pl.direct ? out : nullptr;
  prm.ws_acc = static_cast<float*>(workspace);
  prm.ws_ml = pl.direct ? nullptr
                        : prm.ws_acc + static_cast<size_t>(batch) * num_q_heads * pl.max_parts * head_dim;
  prm.q = q;
  prm.k_pool = k_pool;
  prm.v_pool = v_pool;
  prm.bt = block_tables;
  prm.seq_lens = seq_lens;
  prm.batch = batch;
  prm.mb = max_blocks_per_seq;
  prm.hq = num_q_heads;
  prm.hkv = num_kv_heads;
  prm.group = num_q_heads / num_kv_heads;
  prm.head_groups = prm.group / pl.gt;
  prm.bs_log2 = ilog2(block_size);
  prm.nb = num_blocks;
  prm.window = sliding_window;
  prm.part = pl.part;
  prm.max_parts = pl.max_parts;
  prm.scale_log2 = scale * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(pl.max_parts),
                  static_cast<unsigned>(num_kv_heads * prm.head_groups),
                  static_cast<unsigned>(batch));
  const dim3 block(static_cast<unsigned>(64 * pl.nw));
  {
    LaunchTrace tr(PAGED_KERNEL_DECODE_PARTIAL, s);
    launch_partial_any(prm, esz, head_dim, pl.gt, grid, block, s, tr);
    tr.finish();
    if (int32_t rc = check_launch("paged_attn_decode (partial)")) return rc;
  }
  if (!pl.direct) {
    prm.out = out;
    const dim3 rgrid(static_cast<unsigned>((static_cast<int64_t>(batch) * num_q_heads + 3) / 4));
    LaunchTrace tr(PAGED_KERNEL_DECODE_REDUCE, s);
    if (esz == 2) launch_reduce_d<2>(prm, head_dim, rgrid, s, tr);
    else launch_reduce_d<4>(prm, head_dim, rgrid, s, tr);
    tr.finish();
    if (int32_t rc = check_launch("paged_attn_decode (reduce)")) return rc;
  }
  return ok();
}
