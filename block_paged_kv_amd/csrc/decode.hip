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
// One workgroup handles (row, KV head, group of GT query heads, partition) and
// writes float32 partials (max in log2 units, sum, unnormalised accumulator);
// decode_reduce_kernel combines a row's partitions in partition order, so
// results are deterministic and there are no atomics. When every row fits one
// partition the partial kernel writes the output itself and no reduce runs.
//   * bf16 and FP8 pools (decode_partial_lds_kernel): four waves, each
//     streaming its share of the partition's 16-token K/V stages from the
//     pages straight into a private LDS ring with global_load_lds_dwordx4
//     (streaming cache policy), two stages in flight; S^T = K Q^T and
//     O += P V on the matrix cores; the waves merge through LDS at the end.
//     See the comment above that kernel for the layout.
//   * fp32 pools (decode_partial_kernel): up to four waves on the vector ALU.
//     A token row of K is read by R = 16 (or 8) consecutive lanes with
//     16-byte loads, 16 K and 16 V loads per lane in flight before any is
//     used; q.k is an fp32 FMA chain followed by a DPP sum over the R lanes,
//     so every lane of a row knows the score and the online softmax runs per
//     "token lane"; P.V accumulates in the lane owning those head_dim
//     elements; token lanes, then waves (through LDS), merge at the end.

#include <cmath>
#include <mutex>
#include <vector>

#include "attn.h"
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
  int32_t batch, mb, hq, hkv, group, gt, head_groups, bs_log2, nb, window, part, max_parts;
  float scale_log2;  // scale * log2(e) (times the K scale for FP8 pools)
  float v_scale;     // FP8 pools: the V scale; 1 otherwise
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

  const int hg = blockIdx.x;
  const int b = blockIdx.y;
  const int p = blockIdx.z;
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
// bf16 decode: K/V streamed into LDS by the load unit, both products on MFMA.
//
// Each wave of a workgroup owns a contiguous run of 16-token stages of the
// partition and a private ring of two stage buffers in LDS. A stage's K and V
// rows (16 tokens x head_dim, row-major) are fetched with
// global_load_lds_dwordx4: every lane names its own 16-byte source and the
// data lands at the ring slot's base + 16 * lane, with no registers held and
// no barrier (only the wave itself reads its ring). One stage streams in
// while the other is being computed.
//   * S^T (16 keys x 16 heads) = K Q^T on v_mfma_f32_16x16x32_bf16: the A
//     operand is read from the K rows, the B operand is the query heads of
//     the group (zero beyond GT), held in registers for the whole partition.
//     Lane (lq, lg) receives the scores of head lq for keys 4*lg + i.
//   * O (16 heads x head_dim) += P V on v_mfma_f32_16x16x16_bf16: the S^T
//     accumulator layout is exactly the P operand layout (head lq, keys
//     4*lg .. 4*lg + 3), and the V operand (4 consecutive keys of one head_dim
//     column) comes from the row-major V rows through ds_read_b64_tr_b16.
//     Row sums come from the same product against a ones tile.
//   * Rows are stored in LDS with the 16-byte chunk index XOR-ed by the row
//     index, which spreads the column reads of both products over the banks.
//   * Online softmax in scaled log2 units with lazy rescaling (the reference
//     max moves only when a score exceeds it by 2^8); the partition's
//     (max, sum, accumulator) are exact for whatever reference is kept.
// Stage geometry for head_dim D and KV elements of ESZ bytes (2: bf16,
// 1: FP8 E4M3 codes).
template <int D, int ESZ>
struct StageGeo {
  static constexpr int ROWB = D * ESZ;          // bytes per token row in the pool
  static constexpr int EPC = 16 / ESZ;          // elements per 16-byte chunk
  static constexpr int CPT = ROWB / 16;         // 16-byte chunks per token row
  static constexpr int TPI = 1024 / ROWB;       // token rows per load instruction (1 KiB)
  static constexpr int NI = 16 / TPI;           // load instructions per stage, K (and V)
  static constexpr int SBYTES = 16 * ROWB;      // K (or V) bytes of one stage
  static constexpr int KS = D / 32;             // q.K k-steps
  static constexpr int NT = D / 16;             // output column tiles
  static constexpr int SWZ = CPT < 16 ? CPT - 1 : 15;  // row bits folded into the chunk index
  // bf16 V rows read by the transposing P.V operand load (FP8 stages are
  // widened into such a tile first).
  static constexpr int VROWB = D * 2;
  static constexpr int VSWZ = (VROWB / 16) < 16 ? (VROWB / 16) - 1 : 15;
  // Ring slots per wave: two (one stage landing while the other computes),
  // one at head_dim 512, where a stage of K and V takes 32 KiB and four
  // waves' rings must stay within the compute unit's LDS.
  static constexpr int NSLOT = D >= 512 ? 1 : 2;
  static constexpr int STAGE = 2 * SBYTES;                 // K then V rows of one stage
  static constexpr int WIDE = ESZ == 1 ? 16 * VROWB : 0;   // FP8: the widened V rows
  // Ring slot 0 doubles as the wave-merge buffer (MERGE_ROWS heads x D
  // floats per pass; groups of more heads merge in two passes); with one
  // slot it also holds the widened V rows after the stage. FP8 stages are
  // half the size of bf16 ones, so their merge takes 8 heads per pass and a
  // workgroup's rings stay within 48 KiB at head_dim 128 (three per CU).
  static constexpr int MERGE_ROWS = (ESZ == 1 && D <= 256) ? 8 : 16;
  static constexpr int MERGE = MERGE_ROWS * D * 4;
  static constexpr int SLOT0_DATA = NSLOT == 1 ? STAGE + WIDE : STAGE;
  static constexpr int SLOT0 = SLOT0_DATA > MERGE ? SLOT0_DATA : MERGE;
  // Slot 1 (two slots) or, with one slot, just the merge's (max, sum) rows.
  static constexpr int SLOT1 = NSLOT == 2 ? STAGE : 16 * 2 * 4;
  // LDS reads requested together: every K fragment and V operand of a stage,
  // or (head_dim 512) half of them at a time, to bound the registers.
  static constexpr int KB = KS < 8 ? KS : 8;
  static constexpr int VB = NT < 16 ? NT : 16;
};

constexpr int kStageTokens = 16;
constexpr int kDecodeWaves = 4;

typedef short shortx4d_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8d_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx4_t mfma_k32(const uint4& a, const uint4& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8d_t, a),
                                                 __builtin_bit_cast(bf16x8d_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx4_t mfma_k16(const uint2& a, const uint2& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4d_t, a),
                                                   __builtin_bit_cast(shortx4d_t, b), c, 0, 0, 0);
}


template <int D, int ESZ>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_partial_lds_kernel(DecodeParams a) {
  using Sg = StageGeo<D, ESZ>;
  constexpr bool KV8 = ESZ == 1;
  constexpr int CPT = Sg::CPT, TPI = Sg::TPI, NI = Sg::NI, KS = Sg::KS, NT = Sg::NT;
  constexpr int ROWB = Sg::ROWB, SWZ = Sg::SWZ, EPC = Sg::EPC, SBYTES = Sg::SBYTES;
  constexpr int VROWB = Sg::VROWB, VSWZ = Sg::VSWZ, KB = Sg::KB, VB = Sg::VB;
  constexpr float kNegInf = -INFINITY;

  // One ring slot per array (K rows then V rows), so the compiler can tell the
  // slots apart when it orders LDS reads against the loads still writing
  // other slots. Slot 0 is padded to hold the wave-merge buffer.
  constexpr int NSLOT = Sg::NSLOT;
  __shared__ uint4 ring0[kDecodeWaves][Sg::SLOT0 / 16];
  __shared__ uint4 ring1[kDecodeWaves][Sg::SLOT1 / 16];
  // FP8: each wave's V stage widened to bf16 rows for the transposing read
  // (with one slot, inside slot 0 after the stage).
  constexpr bool WIDE_ARRAY = KV8 && NSLOT == 2;
  __shared__ uint4 vwide[WIDE_ARRAY ? kDecodeWaves : 1][WIDE_ARRAY ? Sg::WIDE / 16 : 1];

  const int hg = blockIdx.x;
  const int b = blockIdx.y;
  const int z = blockIdx.z;
  const int GT = a.gt;
  const int kvh = hg / a.head_groups;
  const int h0 = kvh * a.group + (hg - kvh * a.head_groups) * GT;
  const int n = a.seq_lens[b];
  const int lo = a.window > 0 ? max(0, n - a.window) : 0;
  const int s0 = (lo >> a.bs_log2) << a.bs_log2;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int lq = lane & 15;
  const int lg = lane >> 4;

  const int bs_log2 = a.bs_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const bool bs8 = bs_log2 == 3;
  const int nst_part = a.part / kStageTokens;
  const int spw = (nst_part + nw - 1) / nw;  // stages per wave

  // Query heads h0 .. h0+GT-1 as the B operand of S^T = K Q^T: lane (lq, lg)
  // holds head lq, head_dim elements 32*ks + 8*lg .. +8. Requested before the
  // row length is known, as is (without a window, where a partition's start
  // does not depend on the row length) the wave's first table window.
  uint4 qb[KS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<size_t>(b) * a.hq + h0 + (lq < GT ? lq : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = lq < GT ? *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * lg) : make_uint4(0, 0, 0, 0);
  }
  const int32_t* bt = a.bt + static_cast<size_t>(b) * a.mb;
  const bool spec_tbl = a.window == 0;
  int tbl_first = 0;
  if (spec_tbl) {
    const int lb = ((z * a.part + wave * spw * kStageTokens) >> bs_log2) + lane;
    tbl_first = lb < a.mb ? bt[lb] : 0;
  }
  // A row with fewer partitions than the grid runs its last partition (the
  // partial one) from the grid's last partition slot, and that partition's
  // own slot stays empty: the short partial partitions are then dispatched
  // last and fill the final round of workgroups, where full ones would leave
  // a tail (mixed-length batch 81.8 -> 79.3 us). Decided after the query and
  // the speculative table window are requested, so that the wait for the
  // row length does not hold them back.
  __builtin_amdgcn_sched_barrier(0);
  const int span_row = n - s0;
  int p = z;
  if (z == a.max_parts - 1) {
    if (span_row > 0 && span_row <= z * a.part) p = (span_row - 1) / a.part;
  } else if (span_row > z * a.part && span_row <= (z + 1) * a.part) {
    p = a.max_parts;
  }
  const int ps = s0 + p * a.part;
  if (spec_tbl && p != z && p < a.max_parts) {
    // The moved partition's own first table window.
    const int lb = ((p * a.part + wave * spw * kStageTokens) >> bs_log2) + lane;
    tbl_first = lb < a.mb ? bt[lb] : 0;
  }

  if (ps >= n) {
    // Only an empty row (n == 0) reaches this with p == 0: its output is zero.
    if (a.out && p == 0)
      for (int i = threadIdx.x; i < GT * D; i += blockDim.x)
        store_out<2>(a.out, (static_cast<size_t>(b) * a.hq + h0) * D + i, 0.f);
    return;
  }
  const int t_begin = max(ps, lo);
  const int t_end = min(ps + a.part, n);

  // This wave's stages: a contiguous share of the partition's 16-token
  // stages, clipped to those that touch [t_begin, t_end).
  const int k_first = max(wave * spw, (t_begin - ps) / kStageTokens);
  const int k_last = min(min((wave + 1) * spw, nst_part), (t_end - ps + kStageTokens - 1) / kStageTokens);
  const int nst = max(0, k_last - k_first);  // stages this wave computes
  const int ts0 = ps + k_first * kStageTokens;

  // Block-table window: lane i holds the entry of block tb0 + i.
  const int blk_end = nst > 0 ? ((ts0 + nst * kStageTokens - 1) >> bs_log2) + 1 : 0;
  int tb0 = 0;
  int tbl = 0;
  auto phys_ok = [&](int phys) { return phys > 0 && phys < a.nb; };

  // Lane byte offsets inside a block for each load instruction: the
  // instruction's token row i*TPI + lane/CPT, global chunk (lane%CPT) ^ row.
  uint32_t voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = i * TPI + lane / CPT;
    const int chunk = (lane % CPT) ^ (row & SWZ);
    voff[i] = static_cast<uint32_t>(((row & (bs8 ? 7 : 15)) * D + chunk * EPC) * ESZ);
  }
  // With block size 8 one instruction spans both blocks of a stage only when
  // it covers more than 8 rows (64-byte rows); such stages take the per-lane
  // address form.
  const bool split_rows = bs8 && TPI > 8;
  const char* kpool = static_cast<const char*>(a.k_pool);
  const char* vpool = static_cast<const char*>(a.v_pool);

  // Issue the loads of stage k (0-based within this wave) into the ring slot
  // at LDS offset sl: exactly 2*NI load instructions, every lane active.
  // Returns the stage's valid-token mask (bit t: token ts + t is attended and
  // its block id is valid). The block ids come from the table window, loaded
  // before any stage is in flight. A stage whose 16 rows are all valid loads
  // from the block base (scalar) plus the lane's fixed offset; any other stage
  // gives each lane its own address, rows it does not attend reading the zero
  // chunk.
  auto issue = [&](int k, uint32_t sl) -> uint32_t {
    const int ts = ts0 + k * kStageTokens;
    const int blk = ts >> bs_log2;
    const int phys_lo = __builtin_amdgcn_readlane(tbl, blk - tb0);
    const int phys_hi = __builtin_amdgcn_readlane(tbl, bs8 ? blk + 1 - tb0 : blk - tb0);
    const size_t sub = static_cast<size_t>(ts & bs_mask) * D;
    const size_t base_lo = (((static_cast<size_t>(phys_lo) * a.hkv + kvh) << bs_log2) * D + sub) * ESZ;
    const size_t base_hi = (((static_cast<size_t>(phys_hi) * a.hkv + kvh) << bs_log2) * D + sub) * ESZ;
    const int v0 = min(max(t_begin - ts, 0), kStageTokens);
    const int v1 = min(max(t_end - ts, 0), kStageTokens);
    uint32_t vmask = v1 > v0 ? ((0xFFFFu >> (kStageTokens - v1)) & ~((1u << v0) - 1u)) : 0u;
    if (!phys_ok(phys_lo)) vmask &= bs8 ? 0xFF00u : 0u;
    if (!phys_ok(phys_hi)) vmask &= bs8 ? 0x00FFu : 0u;
    // The slot's previous stage has been consumed; its LDS reads must have
    // returned before the new data lands.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (vmask == 0xFFFFu && !split_rows) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        // With block size 8, rows 8..15 are in the second block.
        const size_t base = (bs8 && i * TPI >= 8) ? base_hi : base_lo;
        lds_dma16_stream(kpool + base, voff[i], sl + i * 1024);
        lds_dma16_stream(vpool + base, voff[i], sl + SBYTES + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = i * TPI + lane / CPT;
        const size_t base = (bs8 && row >= 8) ? base_hi : base_lo;
        const bool ok = (vmask >> row) & 1u;
        const size_t off = base + voff[i];
        const void* ksrc = ok ? static_cast<const void*>(kpool + off) : &kZeroChunk;
        const void* vsrc = ok ? static_cast<const void*>(vpool + off) : &kZeroChunk;
        lds_dma16_stream(ksrc, sl + i * 1024);
        lds_dma16_stream(vsrc, sl + SBYTES + i * 1024);
      }
    }
    return vmask;
  };

  floatx4_t o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  floatx4_t lsum = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float mc = kNegInf;    // reference max of head lq (scaled log2 units)
  float negc = 0.f;
  const uint2 ones = make_uint2(0x3F803F80u, 0x3F803F80u);
  const float c = a.scale_log2;

  auto compute = [&](const uint4* sb, uint32_t vmask) {
    const char* kr = reinterpret_cast<const char*>(sb);
    const char* vr_in = kr + SBYTES;
    // FP8: widen the stage's V rows into this wave's bf16 tile (same row
    // layout as the bf16 kernel reads). Only this wave touches the tile, and a
    // wave's LDS accesses are performed in order.
    const char* vr_bf = vr_in;
    auto k_code_chunk = [&](int ks) { return (2 * ks + (lg >> 1)) ^ (lq & SWZ); };
    uint2 kraw[KV8 && KB == KS ? KS : 1];
    if constexpr (KV8) {
      char* vw = WIDE_ARRAY ? reinterpret_cast<char*>(&vwide[wave][0])
                            : reinterpret_cast<char*>(&ring0[wave][0]) + Sg::STAGE;
      // The stage's K codes (this lane's fragments) and V codes are requested
      // together, ahead of the V tile's widening stores, so one LDS round
      // trip serves both.
      if constexpr (KB == KS) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kraw[ks] = *reinterpret_cast<const uint2*>(kr + lq * ROWB + k_code_chunk(ks) * 16 + 8 * (lg & 1));
      }
      uint4 c8[CPT / 4];
#pragma unroll
      for (int j = 0; j < CPT / 4; ++j) {
        const int q = lane + 64 * j;  // fp8 chunk: row q / CPT, 16 elements (q % CPT)*16 ..
        const int row = q / CPT;
        const int cc = q % CPT;
        c8[j] = *reinterpret_cast<const uint4*>(vr_in + row * ROWB + ((cc ^ (row & SWZ)) << 4));
      }
#pragma unroll
      for (int j = 0; j < CPT / 4; ++j) {
        const int q = lane + 64 * j;
        const int row = q / CPT;
        const int cc = q % CPT;
        const uint4 lo = widen_e4m3x8(make_uint2(c8[j].x, c8[j].y));
        const uint4 hi = widen_e4m3x8(make_uint2(c8[j].z, c8[j].w));
        *reinterpret_cast<uint4*>(vw + row * VROWB + (((2 * cc) ^ (row & VSWZ)) << 4)) = lo;
        *reinterpret_cast<uint4*>(vw + row * VROWB + (((2 * cc + 1) ^ (row & VSWZ)) << 4)) = hi;
      }
      vr_bf = vw;
    }
    // Every LDS read of the stage is requested up front: the A operand of
    // S^T = K Q^T (key lq, head_dim elements 32*ks + 8*lg .. +8) and the B
    // operand of O += P V. For the latter, lane (lq, lg) addresses key row
    // 4*lg + lq/4, columns 16*nt + 4*(lq%4) .. +3; the transposing read
    // returns keys 4*lg .. 4*lg+3 of column 16*nt + lq.
    auto read_k = [&](int ks) -> uint4 {
      if constexpr (KV8) {
        if constexpr (KB == KS) return widen_e4m3x8(kraw[ks]);
        return widen_e4m3x8(*reinterpret_cast<const uint2*>(kr + lq * ROWB + k_code_chunk(ks) * 16 + 8 * (lg & 1)));
      } else {
        const int chunk = (4 * ks + lg) ^ (lq & SWZ);
        return *reinterpret_cast<const uint4*>(kr + lq * ROWB + chunk * 16);
      }
    };
    const int vrow = 4 * lg + (lq >> 2);
    const char* vr = vr_bf + vrow * VROWB + 8 * (lq & 1);
    auto read_v = [&](int nt) -> uint2 {
      const int chunk = (2 * nt + ((lq & 3) >> 1)) ^ (vrow & VSWZ);
      return ds_read_tr16(reinterpret_cast<const uint16_t*>(vr + chunk * 16));
    };
    // ---- S^T = K Q^T --------------------------------------------------------
    floatx4_t s = floatx4_t{0.f, 0.f, 0.f, 0.f};
    uint2 vb[VB];
    if constexpr (KB == KS) {
      // Every K fragment and V operand of the stage requested at once.
      uint4 ka[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[ks] = read_k(ks);
#pragma unroll
      for (int nt = 0; nt < VB; ++nt) vb[nt] = read_v(nt);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s = mfma_k32(ka[ks], qb[ks], s);
    } else {
#pragma unroll
      for (int k0 = 0; k0 < KS; k0 += KB) {
        uint4 ka[KB];
#pragma unroll
        for (int i = 0; i < KB; ++i) ka[i] = read_k(k0 + i);
#pragma unroll
        for (int i = 0; i < KB; ++i) s = mfma_k32(ka[i], qb[k0 + i], s);
      }
    }
    // ---- mask (stages that straddle the range or hold an invalid block) ------
    if (vmask != 0xFFFFu) {
      // The empty asm keeps the per-key tests inside this rarely taken branch.
      uint32_t bits = vmask >> (4 * lg);
      asm volatile("" : "+v"(bits));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!((bits >> i) & 1u)) s[i] = kNegInf;
    }
    // ---- online softmax (lane: head lq, keys ts + 4*lg + i) -----------------
    const float mxc = max_across_groups(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]))) * c;
    if (__any(mxc > mc + 8.f)) {
      const float mnew = fmaxf(mc, mxc);
      const float alpha = mnew == kNegInf ? 1.f : fast_exp2(mc - mnew);
      mc = mnew;
      negc = mnew == kNegInf ? 0.f : -mnew;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * lg + i);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[nt][i] *= al[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) lsum[i] *= al[i];
    }
    uint2 pa;
    pa.x = pack_bf16x2(fast_exp2(fmaf(s[0], c, negc)), fast_exp2(fmaf(s[1], c, negc)));
    pa.y = pack_bf16x2(fast_exp2(fmaf(s[2], c, negc)), fast_exp2(fmaf(s[3], c, negc)));
    // ---- O += P V ---------------------------------------------------------------
    lsum = mfma_k16(pa, ones, lsum);
    if constexpr (VB == NT) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt] = mfma_k16(pa, vb[nt], o[nt]);
    } else {
#pragma unroll
      for (int n0 = 0; n0 < NT; n0 += VB) {
#pragma unroll
        for (int i = 0; i < VB; ++i) vb[i] = read_v(n0 + i);
#pragma unroll
        for (int i = 0; i < VB; ++i) o[n0 + i] = mfma_k16(pa, vb[i], o[n0 + i]);
      }
    }
  };

  // ---- stream: one stage landing while the other computes ------------------
  // Two stages of each wave are in flight at the start of a window; stage
  // k+2 is requested once stage k is consumed. (Requesting stage k+1 only
  // once stage k has landed keeps less in flight and measured faster for
  // 4096-token partitions, slower for the 512-token ones of the mixed batch.)
  // The wave's stages are taken in windows whose blocks fit the 64-entry
  // table register; the pipeline drains at a window's end.
  constexpr int OPS = 2 * NI;  // load instructions per stage
  uint4* const slot0 = &ring0[wave][0];
  uint4* const slot1 = &ring1[wave][0];
  const uint32_t lds0 = lds_offset(slot0);
  const uint32_t lds1 = lds_offset(slot1);
  // Stages per window: an even count whose blocks (plus a block-size
  // misalignment of the first stage) stay within 64 table entries.
  const int spwin = ((63 << bs_log2) / kStageTokens) & ~1;
  for (int w0 = 0; w0 < nst; w0 += spwin) {
    const int w1 = min(nst, w0 + spwin);
    tb0 = (ts0 + w0 * kStageTokens) >> bs_log2;
    if (w0 == 0 && spec_tbl) {
      tbl = tbl_first;  // requested at the start: without a window ts0 = ps + wave * spw * 16
    } else {
      const int lb = tb0 + lane;
      tbl = (lb < blk_end && lb < a.mb) ? bt[lb] : 0;
    }
    vm_wait<0>();  // the window's block ids (and, first time, the query) have arrived
    if constexpr (NSLOT == 2) {
      uint32_t mask0 = issue(w0, lds0);
      uint32_t mask1 = w0 + 1 < w1 ? issue(w0 + 1, lds1) : 0u;
      for (int k = w0; k < w1; k += 2) {
        if (k + 1 < w1) vm_wait<OPS>(); else vm_wait<0>();
        compute(slot0, mask0);
        if (k + 2 < w1) mask0 = issue(k + 2, lds0);
        if (k + 1 < w1) {
          if (k + 2 < w1) vm_wait<OPS>(); else vm_wait<0>();
          compute(slot1, mask1);
          if (k + 3 < w1) mask1 = issue(k + 3, lds1);
        }
      }
    } else {
      // One slot: stage k+1 is requested once stage k has been consumed (its
      // LDS reads returned: issue() waits for them first).
      uint32_t mask0 = issue(w0, lds0);
      for (int k = w0; k < w1; ++k) {
        vm_wait<0>();
        compute(slot0, mask0);
        if (k + 1 < w1) mask0 = issue(k + 1, lds0);
      }
    }
  }

  // ---- merge the waves and store -------------------------------------------
  // Each wave puts its (max, sum) and accumulator rows in its own ring slots
  // (only it has used them), so one barrier suffices before a merge pass; a
  // pass covers MERGE_ROWS query heads.
  constexpr int MR = Sg::MERGE_ROWS;
  static_assert(Sg::SLOT0 >= MR * D * static_cast<int>(sizeof(float)), "merge buffer does not fit");
  static_assert(Sg::SLOT1 >= MR * 2 * static_cast<int>(sizeof(float)), "merge buffer does not fit");
  const float* sm_o = reinterpret_cast<const float*>(ring0);
  const float* sm_ml = reinterpret_cast<const float*>(ring1);
  constexpr int kO = Sg::SLOT0 / 4;      // floats between two waves' accumulator rows
  constexpr int kML = Sg::SLOT1 / 4;     // floats between two waves' (max, sum) rows
  for (int g0 = 0; g0 < GT; g0 += MR) {
    if (g0 > 0) __syncthreads();  // the previous pass has read the buffers
    const int g1 = min(GT, g0 + MR);
    {
      float* my_o = reinterpret_cast<float*>(&ring0[wave][0]);   // [MR][D]
      float* my_ml = reinterpret_cast<float*>(&ring1[wave][0]);  // [MR][2]
      // Lanes holding any of the pass's real rows write all four of theirs
      // (rows up to g0 + MR - 1 stay inside the slot).
      if (4 * lg >= g0 && 4 * lg < g1) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) my_o[(4 * lg - g0 + i) * D + 16 * nt + lq] = o[nt][i];
        if (lq == 0)
#pragma unroll
          for (int i = 0; i < 4; ++i) my_ml[(4 * lg - g0 + i) * 2 + 1] = lsum[i];
      }
      if (lg == 0 && lq >= g0 && lq < g1) my_ml[(lq - g0) * 2] = mc;
    }
    __syncthreads();
    // Four consecutive columns per thread and step: 16-byte LDS reads, one
    // weight computation per four outputs, 8-byte (bf16) or 16-byte (partial)
    // stores. With one wave per SIMD nothing hides per-instruction cost, so
    // the instruction count of this loop is the merge's time.
    constexpr int QD = D / 4;  // column quads per row
    for (int v = threadIdx.x; v < (g1 - g0) * QD; v += blockDim.x) {
      const int gl = v / QD;
      const int g = g0 + gl;
      const int d = (v - gl * QD) * 4;
      // Every wave slot is read at once (all lie inside the rings); the entries
      // of waves past nw, which did not run, are then ignored.
      float mw[kDecodeWaves], lw[kDecodeWaves];
      floatx4_t ow[kDecodeWaves];
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        const float2 ml = *reinterpret_cast<const float2*>(sm_ml + w * kML + gl * 2);
        mw[w] = ml.x;
        lw[w] = ml.y;
        ow[w] = *reinterpret_cast<const floatx4_t*>(sm_o + w * kO + gl * D + d);
      }
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) M = w < nw ? fmaxf(M, mw[w]) : M;
      float L = 0.f;
      floatx4_t A = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        const bool live = w < nw && mw[w] != kNegInf;
        const float f = live ? fast_exp2(mw[w] - M) : 0.f;
        L = live ? fmaf(lw[w], f, L) : L;
#pragma unroll
        for (int e = 0; e < 4; ++e) A[e] = live ? fmaf(ow[w][e], f, A[e]) : A[e];
      }
      const size_t bh = static_cast<size_t>(b) * a.hq + h0 + g;
      if (a.out) {
        // FP8: V codes stand for v_scale * value (1 for bf16: exact)
        const float s = L > 0.f ? a.v_scale / L : 0.f;
        uint2 pk;
        pk.x = pack_bf16x2(A[0] * s, A[1] * s);
        pk.y = pack_bf16x2(A[2] * s, A[3] * s);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + bh * D + d) = pk;
      } else {
        const size_t slot = bh * a.max_parts + p;
#pragma unroll
        for (int e = 0; e < 4; ++e) A[e] *= a.v_scale;
        *reinterpret_cast<floatx4_t*>(a.ws_acc + slot * D + d) = A;
        if (d == 0) {
          a.ws_ml[slot * 2] = M;
          a.ws_ml[slot * 2 + 1] = L;
        }
      }
    }
  }
}


// Partitions per chunk of decode_reduce_kernel with CPT columns per lane: 64
// accumulator registers, 128 from four columns per lane on (one wave then
// covers a pair at head_dim 256 with 16-byte loads; more registers at one or
// two columns per lane measured slower).
constexpr int reduce_chunk(int cpt) { return cpt >= 4 ? 128 / cpt : 64 / cpt; }

// CPT consecutive floats from p (16-, 8- or 4-byte aligned), or zeros.
template <int CPT>
__device__ __forceinline__ void load_cols(float* dst, bool ok, const float* p) {
  if constexpr (CPT % 4 == 0) {
#pragma unroll
    for (int k = 0; k < CPT; k += 4) {
      const floatx4_t v = ok ? *reinterpret_cast<const floatx4_t*>(p + k) : floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[k + e] = v[e];
    }
  } else if constexpr (CPT == 2) {
    const float2 v = ok ? *reinterpret_cast<const float2*>(p) : make_float2(0.f, 0.f);
    dst[0] = v.x;
    dst[1] = v.y;
  } else {
    dst[0] = ok ? *p : 0.f;
  }
}

// CPT consecutive outputs at element index i of out (bf16 for ESZ <= 2, else
// float32), written as one or two wide stores.
template <int ESZ, int CPT>
__device__ __forceinline__ void store_cols(void* out, size_t i, const float* v) {
  if constexpr (ESZ <= 2 && CPT >= 2) {
    uint32_t w[CPT / 2];
#pragma unroll
    for (int k = 0; k < CPT / 2; ++k) w[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
    uint16_t* o = static_cast<uint16_t*>(out) + i;
    if constexpr (CPT == 2) {
      *reinterpret_cast<uint32_t*>(o) = w[0];
    } else {
#pragma unroll
      for (int k = 0; k < CPT / 2; k += 2) *reinterpret_cast<uint2*>(o + 2 * k) = make_uint2(w[k], w[k + 1]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) store_out<ESZ>(out, i + k, v[k]);
  }
}

// Combine each (row, query head) pair's partitions. WPP waves serve one pair
// (a 256-thread workgroup serves 4 / WPP pairs); lane l of the pair's wave w
// owns the CPT = D / (64 WPP) consecutive head_dim columns starting at
// CPT (64 w + l), read and written as one or two wide accesses.
// Partitions are taken in chunks of CH = reduce_chunk(CPT): lane i of
// every wave holds the chunk's partition i (max, sum). The launcher picks the
// fewest waves per pair for which a row's partitions fit one chunk, so that
// the row length, the (max, sum) pairs and every accumulator are requested
// together, before the row's live partition count is known (entries past it
// are fetched but never used, only selected away): one round trip to memory
// before the store. (The kernel also takes further chunks in order, combined
// with an online maximum, but the launcher sends rows with more partitions
// than a chunk to the wide kernel below.) The result does not depend on how
// many empty partitions follow the live ones.
template <int ESZ, int D, int CPT>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeParams a) {
  constexpr float kNegInf = -INFINITY;
  constexpr int WPP = D / (64 * CPT);          // waves per pair
  constexpr int CH = reduce_chunk(CPT);        // partitions per chunk
  static_assert(WPP >= 1 && WPP <= 4 && D == 64 * CPT * WPP, "bad reduce shape");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int h = blockIdx.x * (4 / WPP) + wave / WPP;
  if (h >= a.hq) return;
  const int pair = b * a.hq + h;
  const int c0l = ((wave % WPP) * 64 + lane) * CPT;  // this lane's CPT consecutive columns
  const int P = a.max_parts;
  const float* ml = a.ws_ml + static_cast<size_t>(pair) * P * 2;
  const float* acc = a.ws_acc + static_cast<size_t>(pair) * P * D;

  const int n = a.seq_lens[b];
  // First chunk, requested before anything is waited for.
  float2 mlc = lane < CH && lane < P ? *reinterpret_cast<const float2*>(ml + 2 * lane) : make_float2(kNegInf, 0.f);
  float x[CH][CPT];
#pragma unroll
  for (int u = 0; u < CH; ++u) load_cols<CPT>(x[u], u < P, acc + static_cast<size_t>(u) * D + c0l);

  const int lo = a.window > 0 ? max(0, n - a.window) : 0;
  const int s0 = (lo >> a.bs_log2) << a.bs_log2;
  const int np = n > s0 ? min((n - s0 + a.part - 1) / a.part, P) : 0;

  float o[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) o[k] = 0.f;
  float M = kNegInf, L = 0.f;
  for (int c0 = 0; c0 < np; c0 += CH) {
    if (c0 > 0) {
      // Later chunks (rows with more than CH partitions).
      const int pl = c0 + lane;
      mlc = lane < CH && pl < P ? *reinterpret_cast<const float2*>(ml + 2 * static_cast<size_t>(pl))
                                : make_float2(kNegInf, 0.f);
#pragma unroll
      for (int u = 0; u < CH; ++u) load_cols<CPT>(x[u], c0 + u < P, acc + static_cast<size_t>(c0 + u) * D + c0l);
    }
    const bool live = lane < CH && c0 + lane < np;
    const float mp = live ? mlc.x : kNegInf;
    const float lp = live ? mlc.y : 0.f;
    float cm = mp;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
    const float newM = fmaxf(M, cm);
    // Earlier chunks' sums move to the new reference; empty partitions (max
    // -inf) weigh exactly zero.
    const float f = M == kNegInf ? 0.f : fast_exp2(M - newM);
    const float w = mp == kNegInf ? 0.f : fast_exp2(mp - newM);
    float lw = lp * w;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lw += __shfl_xor(lw, off);
    L = L * f + lw;
#pragma unroll
    for (int k = 0; k < CPT; ++k) o[k] *= f;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const float wu = __shfl(w, u);  // partition c0 + u, held by lane u
      const bool take = c0 + u < np;
#pragma unroll
      for (int k = 0; k < CPT; ++k) o[k] = fmaf(take ? x[u][k] : 0.f, wu, o[k]);
    }
    M = newM;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int k = 0; k < CPT; ++k) o[k] *= inv;
  store_cols<ESZ, CPT>(a.out, static_cast<size_t>(pair) * D + c0l, o);
}

// Rows with more partitions than one chunk of the kernel above holds (64): a
// workgroup per (row, query head, 64 columns), lane
// l owning one column; its four waves take chunks of 64 partitions w, w + 4,
// ... (every wave's first chunk requested before the row length is known),
// each combines its chunks with an online maximum, and the four results are
// combined through LDS. Up to 256 partitions (a 32768-token row alone on
// the device) this is one round trip to memory instead of one per chunk.
template <int ESZ, int D>
__global__ __launch_bounds__(256) void decode_reduce_wide_kernel(DecodeParams a) {
  constexpr float kNegInf = -INFINITY;
  constexpr int kSlices = D / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int pair = blockIdx.x / kSlices;
  const int col = (blockIdx.x - pair * kSlices) * 64 + lane;
  const int b = pair / a.hq;
  const int P = a.max_parts;
  const float* ml = a.ws_ml + static_cast<size_t>(pair) * P * 2;
  const float* acc = a.ws_acc + static_cast<size_t>(pair) * P * D;
  const int nch = (P + 63) / 64;

  float2 mlc = make_float2(kNegInf, 0.f);
  float x[64];
  auto load = [&](int c) {
    const int p0 = c * 64;
    mlc = p0 + lane < P ? *reinterpret_cast<const float2*>(ml + 2 * static_cast<size_t>(p0 + lane))
                        : make_float2(kNegInf, 0.f);
#pragma unroll
    for (int u = 0; u < 64; ++u) x[u] = p0 + u < P ? acc[static_cast<size_t>(p0 + u) * D + col] : 0.f;
  };
  if (wave < nch) load(wave);

  const int n = a.seq_lens[b];
  const int lo = a.window > 0 ? max(0, n - a.window) : 0;
  const int s0 = (lo >> a.bs_log2) << a.bs_log2;
  const int np = n > s0 ? min((n - s0 + a.part - 1) / a.part, P) : 0;

  float M = kNegInf, L = 0.f, o = 0.f;
  for (int c = wave; c < nch && c * 64 < np; c += 4) {
    if (c != wave) load(c);
    const bool live = c * 64 + lane < np;
    const float mp = live ? mlc.x : kNegInf;
    const float lp = live ? mlc.y : 0.f;
    float cm = mp;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
    const float newM = fmaxf(M, cm);
    const float f = M == kNegInf ? 0.f : fast_exp2(M - newM);
    const float w = mp == kNegInf ? 0.f : fast_exp2(mp - newM);
    float lw = lp * w;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lw += __shfl_xor(lw, off);
    L = L * f + lw;
    o *= f;
#pragma unroll
    for (int u = 0; u < 64; ++u) {
      // partition c*64 + u: weight held by lane u (zero past np)
      const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
      o = fmaf(c * 64 + u < np ? x[u] : 0.f, wu, o);
    }
    M = newM;
  }

  __shared__ float sm_m[4], sm_l[4], sm_o[4][64];
  if (lane == 0) {
    sm_m[wave] = M;
    sm_l[wave] = L;
  }
  sm_o[wave][lane] = o;
  __syncthreads();
  if (wave != 0) return;
  float MM = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) MM = fmaxf(MM, sm_m[w]);
  float LL = 0.f, OO = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = sm_m[w];
    const float f = mw == kNegInf ? 0.f : fast_exp2(mw - MM);
    LL = fmaf(sm_l[w], f, LL);
    OO = fmaf(sm_o[w][lane], f, OO);
  }
  store_out<ESZ>(a.out, static_cast<size_t>(pair) * D + col, LL > 0.f ? OO / LL : 0.f);
}

// Tokens one wave of the fp32 kernel processes per iteration.
int iter_tokens_f32(int d) {
  return d == 64 ? Geo<4, 64>::ITER : d == 128 ? Geo<4, 128>::ITER : Geo<4, 256>::ITER;
}

// Query heads one workgroup handles: the largest supported size dividing the
// group (bf16 and FP8 kernel: up to 16, the MFMA row count; fp32 kernel: 4, 2, 1).
int head_group_size(int group, int esz) {
  if (esz <= 2) {
    for (int g = 16; g > 1; --g)
      if (group % g == 0) return g;
    return 1;
  }
  static const int kF32[] = {4, 2, 1};
  for (int g : kF32)
    if (group % g == 0) return g;
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
  if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
    return fail(PAGED_ERR_INVALID_ARG, "head_dim must be 64, 128, 256 or 512 (got %d)", head_dim);
  if (head_dim == 512 && esz > 2)
    return fail(PAGED_ERR_INVALID_ARG, "head_dim 512 needs bf16 or FP8 pools (got float32)");
  if (!pow2_in(block_size, 8, 64))
    return fail(PAGED_ERR_INVALID_ARG, "block_size must be a power of two in [8, 64]");
  if (max_seq_len < 0 || window < 0) return fail(PAGED_ERR_INVALID_ARG, "negative length");
  const int group = hq / hkv;
  pl->gt = head_group_size(group, esz);
  const int32_t span = span_tokens(max_seq_len, window, block_size);
  const int64_t pairs = static_cast<int64_t>(batch) * hkv * (group / pl->gt);
  int32_t part = partition_tokens;
  if (esz <= 2) {
    // Stage-streaming kernel: 16-token stages, four waves per workgroup
    // (two or more workgroups per CU, so one's start and merge overlap
    // another's streaming; eight waves in one workgroup measured slower).
    const int32_t unit = std::max(kStageTokens, block_size);
    if (part == 0) {
      // Aim at every wave slot of the device busy at once (8 waves per CU; 12
      // over FP8 pools up to head_dim 128, whose rings are smaller; 4 at
      // head_dim 256 and 512 where a workgroup's rings take most of the LDS) with
      // whole stages per wave; longer rows get longer partitions.
      const int cus = device_cu_count();
      if (cus <= 0) return fail(PAGED_ERR_HIP, "cannot query the device compute-unit count");
      const int64_t slots = static_cast<int64_t>(head_dim >= 256 ? 4 : (esz == 1 && head_dim <= 128) ? 12 : 8) * cus;
      const int64_t stages = pairs * ((span + kStageTokens - 1) / kStageTokens);
      int64_t spw = std::max<int64_t>(1, (stages + slots - 1) / slots);
      int64_t p2 = 1;
      while (p2 < spw) p2 <<= 1;
      part = static_cast<int32_t>(std::min<int64_t>(p2 * kStageTokens * kDecodeWaves, 65536));
      part = std::max(part, unit);
    }
    if (part < unit || part > 65536 || part % unit != 0)
      return fail(PAGED_ERR_INVALID_ARG,
                  "partition_tokens must be a multiple of %d in [%d, 65536] (got %d)", unit, unit,
                  part);
    // Waves per workgroup depend on the partition size only, so a larger
    // max_seq_len (extra, empty partitions) never changes a row's partials.
    pl->nw = std::min(kDecodeWaves, part / kStageTokens);
  } else {
    if (part == 0) {
      const int cus = device_cu_count();
      if (cus <= 0) return fail(PAGED_ERR_HIP, "cannot query the device compute-unit count");
      part = 64;
      for (int32_t c = 1024; c >= 64; c >>= 1) {
        if (pairs * ((span + c - 1) / c) >= 4LL * cus) {
          part = c;
          break;
        }
      }
      part = std::max(part, block_size);
    }
    if (part < 16 || part > 65536 || part % block_size != 0)
      return fail(PAGED_ERR_INVALID_ARG,
                  "partition_tokens must be a multiple of block_size in [16, 65536] (got %d)", part);
    // Long-lived waves stream best: each wave gets at least 4 iterations of
    // its partition (1..4 waves), a function of the partition size only.
    const int iters = (part + iter_tokens_f32(head_dim) - 1) / iter_tokens_f32(head_dim);
    pl->nw = std::min(kMaxWaves, std::max(1, iters / 4));
  }
  // Partition starts and ends stay well inside 32-bit positions.
  if (static_cast<int64_t>(span) > (int64_t{1} << 30))
    return fail(PAGED_ERR_INVALID_ARG, "max_seq_len (attended span %d) must be at most 2^30 tokens", span);
  pl->part = part;
  pl->max_parts = std::max(1, (span + part - 1) / part);
  pl->direct = pl->max_parts == 1;
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
void launch_partial_stage(const DecodeParams& prm, int kv_esz, dim3 grid, dim3 block,
                          hipStream_t s, const LaunchTrace& tr) {
  if (kv_esz == 1)
    hipExtLaunchKernelGGL(decode_partial_lds_kernel<D, 1>, grid, block, 0, s, tr.start(), tr.stop(), 0, prm);
  else
    hipExtLaunchKernelGGL(decode_partial_lds_kernel<D, 2>, grid, block, 0, s, tr.start(), tr.stop(), 0, prm);
}

// kv_esz: bytes per pool element (4 fp32, 2 bf16, 1 FP8 codes with bf16 q/out).
void launch_partial_any(const DecodeParams& prm, int kv_esz, int d, int gt, dim3 grid, dim3 block,
                        hipStream_t s, const LaunchTrace& tr) {
  if (kv_esz <= 2) {
    if (d == 64) launch_partial_stage<64>(prm, kv_esz, grid, block, s, tr);
    else if (d == 128) launch_partial_stage<128>(prm, kv_esz, grid, block, s, tr);
    else if (d == 256) launch_partial_stage<256>(prm, kv_esz, grid, block, s, tr);
    else launch_partial_stage<512>(prm, kv_esz, grid, block, s, tr);
  } else {
    if (d == 64) launch_partial_f32<64>(prm, gt, grid, block, s, tr);
    else if (d == 128) launch_partial_f32<128>(prm, gt, grid, block, s, tr);
    else launch_partial_f32<256>(prm, gt, grid, block, s, tr);
  }
}

// Waves per (row, query head) of decode_reduce_kernel: the fewest for which a
// row's partitions fit one chunk; 0 when none does (decode_reduce_wide_kernel).
int reduce_waves_per_pair(int d, int max_parts) {
  for (int wpp = 1; wpp <= 4; wpp *= 2) {
    const int cpt = d / (64 * wpp);
    if (cpt >= 1 && max_parts <= reduce_chunk(cpt)) return wpp;
  }
  return 0;
}

template <int ESZ, int D>
void launch_reduce_w(const DecodeParams& prm, int wpp, hipStream_t s, const LaunchTrace& tr) {
  const dim3 block(256);
  auto go = [&](auto kern, int pairs_per_wg) {
    const dim3 grid(static_cast<unsigned>((prm.hq + pairs_per_wg - 1) / pairs_per_wg),
                    static_cast<unsigned>(prm.batch));
    hipExtLaunchKernelGGL(kern, grid, block, 0, s, tr.start(), tr.stop(), 0, prm);
  };
  if constexpr (D == 64) {
    go(decode_reduce_kernel<ESZ, 64, 1>, 4);
  } else if constexpr (D == 128) {
    if (wpp == 1) go(decode_reduce_kernel<ESZ, 128, 2>, 4);
    else go(decode_reduce_kernel<ESZ, 128, 1>, 2);
  } else if constexpr (D == 256) {
    if (wpp == 1) go(decode_reduce_kernel<ESZ, 256, 4>, 4);
    else if (wpp == 2) go(decode_reduce_kernel<ESZ, 256, 2>, 2);
    else go(decode_reduce_kernel<ESZ, 256, 1>, 1);
  } else {
    if (wpp == 1) go(decode_reduce_kernel<ESZ, 512, 8>, 4);
    else if (wpp == 2) go(decode_reduce_kernel<ESZ, 512, 4>, 2);
    else go(decode_reduce_kernel<ESZ, 512, 2>, 1);
  }
}

template <int ESZ, int D>
void launch_reduce_wide(const DecodeParams& prm, hipStream_t s, const LaunchTrace& tr) {
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(prm.batch) * prm.hq * (D / 64)));
  hipExtLaunchKernelGGL(decode_reduce_wide_kernel<ESZ, D>, grid, dim3(256), 0, s, tr.start(), tr.stop(), 0,
                        prm);
}

template <int ESZ>
void launch_reduce_d(const DecodeParams& prm, int d, hipStream_t s, const LaunchTrace& tr) {
  const int wpp = reduce_waves_per_pair(d, prm.max_parts);
  if (wpp == 0) {
    if (d == 64) launch_reduce_wide<ESZ, 64>(prm, s, tr);
    else if (d == 128) launch_reduce_wide<ESZ, 128>(prm, s, tr);
    else if (d == 256) launch_reduce_wide<ESZ, 256>(prm, s, tr);
    else if constexpr (ESZ == 2) launch_reduce_wide<ESZ, 512>(prm, s, tr);
    return;
  }
  if (d == 64) launch_reduce_w<ESZ, 64>(prm, wpp, s, tr);
  else if (d == 128) launch_reduce_w<ESZ, 128>(prm, wpp, s, tr);
  else if (d == 256) launch_reduce_w<ESZ, 256>(prm, wpp, s, tr);
  else if constexpr (ESZ == 2) launch_reduce_w<ESZ, 512>(prm, wpp, s, tr);
}

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

extern "C" int32_t paged_attn_decode_partition_tokens(int32_t batch, int32_t num_q_heads,
                                                      int32_t num_kv_heads, int32_t head_dim,
                                                      int32_t block_size, int32_t max_seq_len,
                                                      int32_t sliding_window, int32_t dtype,
                                                      int32_t* partition_tokens) {
  if (!partition_tokens) return fail(PAGED_ERR_INVALID_ARG, "NULL argument");
  const int esz = esize_of(dtype);
  if (esz == 0) return fail(PAGED_ERR_DTYPE, "unknown dtype %d", dtype);
  Plan pl;
  if (int32_t rc = make_plan(batch, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len,
                             sliding_window, 0, esz, &pl))
    return rc;
  *partition_tokens = pl.part;
  return ok();
}

extern "C" int32_t paged_attn_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                                     int32_t num_kv_heads, int32_t head_dim,
                                                     int32_t block_size, int32_t max_seq_len,
                                                     int32_t sliding_window,
                                                     int32_t partition_tokens, int32_t dtype,
                                                     size_t* bytes) {
  if (!bytes) return fail(PAGED_ERR_INVALID_ARG, "NULL argument");
  const int esz = esize_of(dtype);
  if (esz == 0) return fail(PAGED_ERR_DTYPE, "unknown dtype %d", dtype);
  Plan pl;
  if (int32_t rc = make_plan(batch, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len,
                             sliding_window, partition_tokens, esz, &pl))
    return rc;
  *bytes = pl.ws_bytes;
  return ok();
}

namespace pagedkv {

namespace {

int32_t decode_check_plan(const void* out, const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, float scale, float k_scale, float v_scale,
                          int32_t sliding_window, int32_t partition_tokens, int32_t max_seq_len,
                          const void* workspace, size_t workspace_bytes, int esz, Plan* pl) {
  if (int32_t rc = make_plan(batch, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len,
                             sliding_window, partition_tokens, esz, pl))
    return rc;
  if (max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(PAGED_ERR_INVALID_ARG, "max_blocks_per_seq and num_blocks must be positive");
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(PAGED_ERR_INVALID_ARG, "scale must be finite and positive");
  if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(PAGED_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if (batch > 65535 || num_q_heads > 65535)
    return fail(PAGED_ERR_INVALID_ARG, "batch and num_q_heads must be at most 65535");
  if (static_cast<int64_t>(batch) * num_q_heads > (1 << 24))
    return fail(PAGED_ERR_INVALID_ARG, "batch * num_q_heads must be at most 2^24");
  if (pl->max_parts > 65535)
    return fail(PAGED_ERR_INVALID_ARG,
                "max_seq_len %d needs %d partitions of %d tokens; at most 65535 are supported",
                max_seq_len, pl->max_parts, pl->part);
  if (batch == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !seq_lens)
    return fail(PAGED_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PAGED_ERR_INVALID_ARG, "misaligned pointer");
  if (!pl->direct) {
    if (!workspace || !aligned16(workspace))
      return fail(PAGED_ERR_INVALID_ARG, "workspace is NULL or misaligned");
    if (workspace_bytes < pl->ws_bytes)
      return fail(PAGED_ERR_CAPACITY, "workspace needs %zu bytes, got %zu", pl->ws_bytes,
                  workspace_bytes);
  }
  return ok();
}

}  // namespace

int32_t decode_check(const void* out, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, float scale, float k_scale, float v_scale,
                     int32_t sliding_window, int32_t partition_tokens, int32_t max_seq_len,
                     const void* workspace, size_t workspace_bytes, int esz) {
  Plan pl;
  return decode_check_plan(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, seq_lens,
                           batch, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                           scale, k_scale, v_scale, sliding_window, partition_tokens, max_seq_len,
                           workspace, workspace_bytes, esz, &pl);
}

// Shared by the bf16/fp32 and the FP8 entry points and the mixed step. esz:
// pool element bytes (q/out are bf16 when esz == 1).
int32_t decode_impl(void* out, const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, float scale, float k_scale, float v_scale,
                    int32_t sliding_window, int32_t partition_tokens, int32_t max_seq_len,
                    void* workspace, size_t workspace_bytes, int esz, void* stream) {
  Plan pl;
  if (int32_t rc = decode_check_plan(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                                     seq_lens, batch, num_q_heads, num_kv_heads, head_dim,
                                     block_size, num_blocks, scale, k_scale, v_scale,
                                     sliding_window, partition_tokens, max_seq_len, workspace,
                                     workspace_bytes, esz, &pl))
    return rc;
  if (batch == 0) return ok();
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
  prm.gt = pl.gt;
  prm.head_groups = prm.group / pl.gt;
  prm.bs_log2 = ilog2(block_size);
  prm.nb = num_blocks;
  prm.window = sliding_window;
  prm.part = pl.part;
  prm.max_parts = pl.max_parts;
  prm.scale_log2 = scale * 1.4426950408889634f * k_scale;
  prm.v_scale = v_scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Partition index slowest: a row whose span is shorter than max_seq_len
  // leaves its later partitions empty, and those workgroups (which only read
  // the row length before leaving) are then dispatched together near the end
  // instead of holding slots between the streaming ones; the bf16 and FP8
  // kernel also runs such a row's last, partial partition from the last slot.
  const dim3 grid(static_cast<unsigned>(num_kv_heads * prm.head_groups),
                  static_cast<unsigned>(batch),
                  static_cast<unsigned>(pl.max_parts));
  const dim3 block(static_cast<unsigned>(64 * pl.nw));
  {
    LaunchTrace tr(PAGED_KERNEL_DECODE_PARTIAL, s);
    launch_partial_any(prm, esz, head_dim, pl.gt, grid, block, s, tr);
    tr.finish();
    if (int32_t rc = check_launch("paged_attn_decode (partial)")) return rc;
  }
  if (!pl.direct) {
    prm.out = out;
    LaunchTrace tr(PAGED_KERNEL_DECODE_REDUCE, s);
    if (esz <= 2) launch_reduce_d<2>(prm, head_dim, s, tr);  // bf16 output
    else launch_reduce_d<4>(prm, head_dim, s, tr);
    tr.finish();
    if (int32_t rc = check_launch("paged_attn_decode (reduce)")) return rc;
  }
  return ok();
}

}  // namespace pagedkv

extern "C" int32_t paged_attn_decode(void* out, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                     int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     float scale, int32_t sliding_window,
                                     int32_t partition_tokens, int32_t max_seq_len,
                                     void* workspace, size_t workspace_bytes, int32_t dtype,
                                     void* stream) {
  if (dtype != PAGED_F32 && dtype != PAGED_BF16)
    return fail(PAGED_ERR_DTYPE, "paged_attn_decode takes f32 or bf16 (FP8 pools: paged_attn_decode_fp8), got %d",
                dtype);
  return decode_impl(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, seq_lens, batch,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, 1.f, 1.f,
                     sliding_window, partition_tokens, max_seq_len, workspace, workspace_bytes,
                     esize_of(dtype), stream);
}

extern "C" int32_t paged_attn_decode_fp8(void* out, const void* q, const void* k_pool,
                                         const void* v_pool, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                         int32_t batch, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t block_size, int32_t num_blocks, float scale,
                                         float k_scale, float v_scale, int32_t sliding_window,
                                         int32_t partition_tokens, int32_t max_seq_len,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, seq_lens, batch,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, k_scale,
                     v_scale, sliding_window, partition_tokens, max_seq_len, workspace,
                     workspace_bytes, 1, stream);
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace: the split-K partials live in a
// file-scope device array, one copy per GPU for the life of the process.
namespace pagedkv {
namespace {

constexpr size_t kScratchBytes = size_t{16} << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this GPU's `scratch`, looked up once per device with that
// device current (host code must never pass the array's own name to a kernel:
// on the host it is a stand-in, not a device address).
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;

int32_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PAGED_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (static_cast<int>(g_scratch_ptr.size()) <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PAGED_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

}  // namespace
}  // namespace pagedkv

extern "C" int32_t paged_attn_decode_noalloc(void* out, const void* q, const void* k_pool,
                                             const void* v_pool, const int32_t* block_tables,
                                             int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                             int32_t batch, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t num_blocks, float scale,
                                             int32_t sliding_window, int32_t partition_tokens,
                                             int32_t max_seq_len, int32_t dtype, void* stream) {
  if (dtype != PAGED_F32 && dtype != PAGED_BF16)
    return fail(PAGED_ERR_DTYPE, "paged_attn_decode_noalloc takes f32 or bf16, got %d", dtype);
  size_t need = 0;
  if (int32_t rc = paged_attn_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                     block_size, max_seq_len, sliding_window,
                                                     partition_tokens, dtype, &need))
    return rc;
  if (need > kScratchBytes)
    return fail(PAGED_ERR_CAPACITY,
                "paged_attn_decode_noalloc: these arguments need %zu bytes of partials, more than "
                "the library's %zu-byte device scratch (use paged_attn_decode with a workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0)
    if (int32_t rc = scratch_address(&ws)) return rc;
  return decode_impl(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, seq_lens, batch,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, 1.f, 1.f,
                     sliding_window, partition_tokens, max_seq_len, ws, need > 0 ? kScratchBytes : 0,
                     esize_of(dtype), stream);
}
