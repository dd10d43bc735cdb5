// Chunked-prefill attention over a block-paged cache, bf16 MFMA (gfx950).
//
// What is computed (mlx-node perf doc, paged-attention knobs table: prefill
// chunk size and the bridge that reads prefill K/V through the pages): every
// query of a chunk at absolute position a = P + i attends, with plain softmax,
// to the keys [lo, a] of its request, K/V read in place through the request's
// block table; the chunk's own K/V was written first.
//
// How (ours):
//   * Query rows are (position, query head) pairs of one KV head, packed
//     position-major, so the G query heads sharing a KV head share every K/V
//     tile. A wave owns 32 rows up to head_dim 128 and 16 beyond; a
//     workgroup has eight waves. At head_dim 512 the waves come in pairs
//     over the same 16 rows, each holding half of head_dim.
//   * K/V tiles of 128 keys (bf16 up to head_dim 128), 64 (others) or 32
//     (head_dim 512) are staged in LDS, both
//     row-major (key, head_dim); the P.V operand is read with a transposing
//     LDS read (ds_read_b64_tr_b16), which hands each lane consecutive keys.
//     Operand reads run a few fragments ahead of the products.
//   * S^T = K Q^T and O += P V run on v_mfma_f32_16x16x32_bf16 with fp32
//     accumulators; the S^T accumulator layout (one query per lane, 4 keys per
//     register group) is exactly the A-operand layout P needs, once converted
//     to bf16, so no shuffle sits between the two products.
//   * Online softmax in fp32 (log2 units); the causal / window mask is applied
//     only on tiles that straddle a row's range.
//   * The 1-D grid is remapped so consecutive tiles of one KV head land on one
//     XCD (round-robin dispatch puts workgroup i on XCD i % 8): that XCD's L2
//     then serves the head's K/V to all of its tiles.

#include <cmath>

#include "attn.h"
#include "device.h"
#include "runtime.h"

namespace pagedkv {
namespace {

// Query rows per wave: 32 (two 16-row MFMA tiles) up to head_dim 128, 16 from
// head_dim 256, where two tiles' accumulators would leave one wave per SIMD.
constexpr int rows_per_wave(int d) { return d >= 256 ? 16 : 32; }
// Keys per K/V tile. 128 for bf16 pools up to head_dim 128: the
// double-buffered K and V tiles take 128 KiB of LDS, and half as many tiles
// per row halve the barriers and per-tile softmax bookkeeping (the
// 2048-token chunk over a 63488-token prefix 1.90 -> 1.82 ms). 64 otherwise:
// FP8 staging registers spill at 128 (measured 1.7x slower), and at head_dim
// 256 two 128-key buffers would not fit the LDS. 32 at head_dim 512, where
// two buffers of 64 one-KiB key rows (K and V) would not fit in a CU's 160 KiB.
constexpr int tile_keys(int d, int esz) { return d >= 512 ? 32 : (d <= 128 && esz == 2) ? 128 : 64; }
// Waves that share a set of query rows and split the head dimension between
// them: two at head_dim 512, one below. Each of the two holds half of the
// query operands, computes the partial scores over its half, exchanges them
// with its partner through LDS, and accumulates half of the output columns:
// the accumulators of 16 rows x 256 columns and half the query operands fit
// two waves per SIMD, where one wave holding all 512 columns needed the
// whole register file of its SIMD.
constexpr int splits(int d) { return d >= 512 ? 2 : 1; }
// Waves per workgroup: eight (up to head_dim 128, 256 query rows share each
// staged K/V tile and the workgroup fills a CU's registers; at head_dim 256,
// 8 x 16 rows, two waves per SIMD, the 128 KiB of tiles allow one workgroup;
// at 512, four pairs of waves over 64 rows). Beside the decode of the mixed
// step too: four-wave workgroups with 64-key tiles, two per CU so that decode
// workgroups fit beside one of them, measured 2% slower there.
constexpr int kPrefillWaves = 8;
constexpr int kNumXcd = 8;

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

struct PrefillParams {
  uint16_t* out;
  const uint16_t* q;
  const void* k_pool;       // bf16 values or FP8 E4M3 codes
  const void* v_pool;
  const int32_t* bt;
  const int32_t* cu_q;
  const int32_t* seq_lens;
  int32_t mb, hq, hkv, group, bs_log2, nb, window;
  int32_t tiles_per_head;   // ceil(max_q_len * group / query rows per workgroup)
  int32_t ksplit;           // key ranges per query tile (1: the whole range, output directly)
  int32_t work_items;       // batch * hkv * ksplit * tiles_per_head
  int32_t per_xcd;          // ceil(work_items / kNumXcd)
  int32_t total_q;
  int32_t last_first;       // 1: a row's query tiles run last-first (see the kernel)
  float scale_log2;         // scale * log2(e) (times the K scale for FP8 pools)
  float v_scale;            // FP8 pools: the V scale; 1 otherwise
  // ksplit > 1: per key range s, query token t, query head h the unnormalised
  // output (times v_scale) at ws_acc[((s * total_q + t) * hq + h) * D] and
  // (reference max in scaled log2 units, probability sum) at ws_ml[... * 2].
  float* ws_acc;
  float* ws_ml;
};

__device__ __forceinline__ floatx4_t mfma16x16x32(const uint4& a, const uint4& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a),
                                                 __builtin_bit_cast(bf16x8v, b), c, 0, 0, 0);
}

// ESZ: bytes per pool element (2: bf16; 1: FP8 E4M3 codes, widened to bf16
// exactly as they are staged, so everything after staging is shared).
template <int D, int ESZ, int NW>
__global__ __launch_bounds__(NW * 64, 1) void prefill_kernel(PrefillParams a) {
  constexpr int kWaves = NW;
  constexpr int SPL = splits(D);    // waves per set of query rows
  constexpr int RG = NW / SPL;      // row groups of the workgroup
  constexpr int RPW = rows_per_wave(D);
  constexpr int JT = RPW / 16;  // 16-row query tiles per wave
  constexpr int kTileM = RG * RPW;
  constexpr int kTileN = tile_keys(D, ESZ);
  constexpr int NS = kTileN / 16;    // 16-key sub-tiles per tile (S^T column tiles)
  constexpr int NK = kTileN / 32;    // 32-key MFMA steps of P.V per tile
  // LDS tiles: key rows of D bf16 elements, unpadded; the 16-byte chunks of
  // a row are stored XOR-swizzled (chunk c of row r at position c ^ swz(r))
  // so that both read patterns below are free of bank conflicts: K reads 16
  // rows x one 16-byte chunk per ds_read_b128 (swz_k: a distinct position
  // per row of a 16-row group), V reads 8 rows x 32 contiguous bytes per
  // half-wave ds_read_b64_tr_b16 (swz_v: even values, so a row's chunk pair
  // stays together and the 8 rows' pairs are distinct). With 128-byte rows
  // (head_dim 64) two rows share a bank line and the row's low bit is
  // folded out.
  constexpr int DCH = D / 8;         // 16-byte chunks per key row
  constexpr int KS = D / 32;         // MFMA k-steps over head_dim
  constexpr int NT = D / 16;         // output column tiles
  constexpr int KSW = KS / SPL;      // k-steps of this wave's part of head_dim
  constexpr int NTW = NT / SPL;      // output column tiles of this wave
  constexpr int ROWB = D * 2;        // bytes per LDS key row
  constexpr float kNegInf = -INFINITY;
  auto swz_k = [](int r) { return D >= 128 ? (r & 15) : ((r >> 1) & 7); };
  auto swz_v = [](int r) { return D >= 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); };

  __shared__ __attribute__((aligned(16))) uint16_t k_s[2][kTileN * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_s[2][kTileN * D];
  // Partial scores handed to the partner wave (split head dimension only).
  __shared__ floatx4_t exch[SPL > 1 ? NW : 1][SPL > 1 ? JT * (kTileN / 16) : 1][64];

  // XCD-aware work mapping: XCD x takes work items [x*per_xcd, (x+1)*per_xcd).
  const int lin = blockIdx.x;
  const int item = (lin % kNumXcd) * a.per_xcd + lin / kNumXcd;
  if (item >= a.work_items) return;
  // Query tile fastest, then key range: consecutive items (one XCD) read the
  // same keys of one KV head. With last_first, a row's tiles run last-first:
  // later query positions attend more keys, so the longest tiles start first
  // and the shortest fill the last round (hybrid prefill 341 -> 328 us per
  // layer). Beside the decode of the mixed step the order stays first-first
  // (last-first there: no faster with bf16 pools, 0.3% slower over FP8).
  const int tile = a.last_first ? a.tiles_per_head - 1 - item % a.tiles_per_head : item % a.tiles_per_head;
  const int rest = item / a.tiles_per_head;
  const int ksp = rest % a.ksplit;
  const int kvh = (rest / a.ksplit) % a.hkv;
  const int b = rest / (a.ksplit * a.hkv);

  const int q0 = a.cu_q[b];
  const int C = a.cu_q[b + 1] - q0;
  const int n = a.seq_lens[b];
  const int P = n - C;
  const int G = a.group;
  const int rows = C * G;
  const int r_first = tile * kTileM;
  if (r_first >= rows || P < 0) return;
  const int r_last = min(r_first + kTileM, rows) - 1;
  const int a_min = P + r_first / G;
  const int a_max = P + r_last / G;
  const int lo_min = a.window > 0 ? max(0, a_min - a.window + 1) : 0;
  const int lo_max = a.window > 0 ? max(0, a_max - a.window + 1) : 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 15;   // query column inside a 16-wide tile
  const int lg = lane >> 4;   // lane group 0..3
  const int wrow = SPL > 1 ? wave % RG : wave;  // this wave's set of query rows
  const int half = SPL > 1 ? wave / RG : 0;     // its part of head_dim

  // Query rows of this lane in the S^T layout: wave rows 16j + lq.
  int qpos[JT], qlo[JT];
  bool qvalid[JT];
  uint4 qreg[JT][KSW];
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    const int r = r_first + wrow * RPW + 16 * j + lq;
    qvalid[j] = r <= r_last;
    const int pos = qvalid[j] ? r / G : 0;
    const int g = qvalid[j] ? r - pos * G : 0;
    qpos[j] = P + pos;
    qlo[j] = a.window > 0 ? max(0, qpos[j] - a.window + 1) : 0;
    const uint16_t* qrow = a.q + (static_cast<size_t>(q0 + pos) * a.hq + kvh * G + g) * D;
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks)
      qreg[j][ks] = qvalid[j] ? *reinterpret_cast<const uint4*>(qrow + (half * KSW + ks) * 32 + lg * 8)
                              : make_uint4(0, 0, 0, 0);
  }

  floatx4_t o[JT][NTW];
#pragma unroll
  for (int j = 0; j < JT; ++j)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) o[j][nt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  // Reference max per query row in scaled log2 units (scale > 0, so the max
  // of the raw scores scales to it), and its negation for the exponent.
  float mc[JT], negc[JT];
  // Row sums accumulate on the matrix core: P times a ones tile gives, in the
  // O layout, the sum of the same bf16 probabilities the numerator uses.
  floatx4_t lsum[JT];
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    mc[j] = kNegInf;
    negc[j] = 0.f;
    lsum[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);

  const int32_t* bt = a.bt + static_cast<size_t>(b) * a.mb;
  const int bs_log2 = a.bs_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  // Key tiles of the workgroup's rows; with a key split, range ksp of ksplit
  // near-equal ranges of them (possibly empty: the partials then say so).
  int kt_begin = lo_min / kTileN;
  int kt_end = a_max / kTileN;  // inclusive
  if (a.ksplit > 1) {
    const int nkt = kt_end - kt_begin + 1;
    const int k0 = kt_begin + nkt * ksp / a.ksplit;
    kt_end = kt_begin + nkt * (ksp + 1) / a.ksplit - 1;
    kt_begin = k0;
  }
  // Blocks a K/V tile touches: a 32-key tile lies inside one 64-key block.
  const int tile_blocks = max(1, kTileN >> bs_log2);
  const float c = a.scale_log2;

  // Block-table entries of one tile, one per lane (lane < tile_blocks).
  auto load_entries = [&](int kt) -> int {
    const int lb = ((kt * kTileN) >> bs_log2) + lane;
    return (kt <= kt_end && lane < tile_blocks && lb < a.mb && (lb << bs_log2) < n) ? bt[lb] : 0;
  };
  auto phys_ok = [&](int phys) { return phys > 0 && phys < a.nb; };

  // Staging (double buffered): wave w moves keys KPW*w .. KPW*w + KPW-1 of a
  // tile, K and V alike. bf16 pools go straight to LDS (global_load_lds_dwordx4: one
  // instruction fills 1 KiB, i.e. RPI consecutive key rows; each lane names
  // the global chunk that belongs at its swizzled LDS position), so no
  // registers hold the next tile. FP8 pools are read into registers, widened
  // to bf16 and stored at the same swizzled positions.
  // The wave's keys lie in one block, or in two when 16 keys meet block_size
  // 8 (keys 8..15 in the second): block ids come from the tile's
  // entries by readlane, so block bases are wave-uniform and each lane adds a
  // loop-invariant 32-bit offset.
  constexpr int RPI = 64 / DCH;                   // key rows per load instruction
  constexpr int KPW = kTileN / kWaves;            // keys each wave stages (4 to 16)
  constexpr int KI = KPW / RPI;                   // load instructions per wave per tile (K, and V)
  const bool bs8 = bs_log2 == 3;
  const bool split = bs8 && KPW > 8;              // the wave's keys span two blocks
  const int lrow = lane / DCH;                    // row inside the instruction
  const int lch = lane % DCH;                     // LDS chunk position inside the row
  uint32_t koff[KI], voff[KI];                    // byte offsets inside the wave's block(s)
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int r = RPI * i + lrow;                 // key row among the wave's KPW
    const int tr = wave * KPW + r;                // tile row (the swizzles use its low bits)
    const int in_blk = split ? (r & 7) : r;
    koff[i] = static_cast<uint32_t>((in_blk * D + (lch ^ swz_k(tr)) * 8) * ESZ);
    voff[i] = static_cast<uint32_t>((in_blk * D + (lch ^ swz_v(tr)) * 8) * ESZ);
  }
  uint2 kraw[ESZ == 1 ? KI : 1], vraw[ESZ == 1 ? KI : 1];  // FP8: codes awaiting their widening store
  const char* kpool = static_cast<const char*>(a.k_pool);
  const char* vpool = static_cast<const char*>(a.v_pool);
  // Returns the tile's absent-block mask: bit i set when the tile's i-th
  // block holds keys of the row (below n) but its table entry is not a valid
  // block id (0, >= num_blocks, or a column past max_blocks_per_seq). Those
  // keys are staged as zeros and masked out of the softmax, as in decode.
  auto stage_load = [&](int kt, int ent, int buf) -> uint64_t {
    const int ts = kt * kTileN;
    const int lb_tile = (ts >> bs_log2) + lane;
    const uint64_t absent = __ballot(lane < tile_blocks && (lb_tile << bs_log2) < n && !phys_ok(ent));
    const int e0 = (wave * KPW) >> bs_log2;
    const int phys_lo = __builtin_amdgcn_readlane(ent, e0);
    const int phys_hi = __builtin_amdgcn_readlane(ent, split ? e0 + 1 : e0);
    // Byte offset of the wave's first key row inside its block (0 unless block_size > 16).
    const size_t sub = static_cast<size_t>((ts + wave * KPW) & bs_mask) * D;
    const size_t base_lo = (((static_cast<size_t>(phys_lo) * a.hkv + kvh) << bs_log2) * D + sub) * ESZ;
    const size_t base_hi = (((static_cast<size_t>(phys_hi) * a.hkv + kvh) << bs_log2) * D + sub) * ESZ;
    const bool full = ts + kTileN <= n && phys_ok(phys_lo) && phys_ok(phys_hi);
    if constexpr (ESZ == 2) {
      const uint32_t kl = lds_offset(&k_s[buf][0]) + wave * KPW * ROWB;
      const uint32_t vl = lds_offset(&v_s[buf][0]) + wave * KPW * ROWB;
      // The buffer's previous tile was read before the last barrier; this
      // wave's own reads of it have returned too.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (full) {
        // Every key of the tile exists and every block id is valid.
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          const size_t base = (split && RPI * i >= 8) ? base_hi : base_lo;
          lds_dma16(kpool + base, koff[i], kl + i * 1024);
          lds_dma16(vpool + base, voff[i], vl + i * 1024);
        }
      } else {
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          const int r = RPI * i + lrow;
          const bool hi = split && r >= 8;
          const bool ok = ts + wave * KPW + r < n && phys_ok(hi ? phys_hi : phys_lo);
          const size_t base = hi ? base_hi : base_lo;
          lds_dma16(ok ? static_cast<const void*>(kpool + base + koff[i]) : &kZeroChunk, kl + i * 1024);
          lds_dma16(ok ? static_cast<const void*>(vpool + base + voff[i]) : &kZeroChunk, vl + i * 1024);
        }
      }
    } else {
      // Every load is issued before any is used; absent rows read the zero chunk.
      if (full) {
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          const size_t base = (split && RPI * i >= 8) ? base_hi : base_lo;
          kraw[i] = *reinterpret_cast<const uint2*>(kpool + base + koff[i]);
          vraw[i] = *reinterpret_cast<const uint2*>(vpool + base + voff[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          const int r = RPI * i + lrow;
          const bool hi = split && r >= 8;
          const bool ok = ts + wave * KPW + r < n && phys_ok(hi ? phys_hi : phys_lo);
          const size_t base = hi ? base_hi : base_lo;
          kraw[i] = *reinterpret_cast<const uint2*>(ok ? static_cast<const void*>(kpool + base + koff[i]) : &kZeroChunk);
          vraw[i] = *reinterpret_cast<const uint2*>(ok ? static_cast<const void*>(vpool + base + voff[i]) : &kZeroChunk);
        }
      }
    }
    return absent;
  };
  // Completes the staging of buffer `buf` for this wave: the direct loads
  // have landed (bf16), or the widened registers are stored (FP8). A barrier
  // must follow before any wave reads the tile.
  auto stage_store = [&](int buf) {
    if constexpr (ESZ == 2) {
      vm_wait<0>();
    } else {
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const int row = wave * KPW + RPI * i + lrow;
        *reinterpret_cast<uint4*>(&k_s[buf][row * D + lch * 8]) = widen_e4m3x8(kraw[i]);
        *reinterpret_cast<uint4*>(&v_s[buf][row * D + lch * 8]) = widen_e4m3x8(vraw[i]);
      }
    }
  };

  // One K/V tile in three parts: S^T = K Q^T (matrix core), the online
  // softmax (vector ALU), O += P V (matrix core). A score array carries the
  // first part's result to the second, pa the probabilities to the third.
  typedef floatx4_t Scores[JT][NS];
  uint4 pa[JT][NK];  // P as bf16 A operands: [query tile][32-key step]

  // ---- S^T = K Q^T over the tile's NS key sub-tiles x JT query tiles ----------
  // The swizzle changes only the low four bits of a chunk index, so chunk
  // 4ks + lg = 16 (ks / 4) + (4 (ks % 4) + lg) lands at 16 (ks / 4) plus one of
  // four lane-dependent positions: the rest is an immediate offset.
  // The K fragment reads run PF fragments ahead of the products and the key
  // sub-tiles' accumulation chains alternate; scheduling barriers keep that
  // order (left to itself the compiler waits on each read right before its
  // product, which a second wave on the SIMD can only partly hide). Eight
  // ahead from head_dim 256, where the waves wait on LDS results and the
  // registers allow it, four below. With the
  // head dimension split, the wave's k-steps start at half * KSW: whole
  // groups of four, so the half only moves the row base.
  auto tile_s = [&](Scores& sc, const uint16_t* ks_buf) {
    const uint16_t* krow = ks_buf + lq * D + half * (KSW / 4) * 128;
    auto kfrag = [&](int t4, int ks) {
      const int pos = (((4 * (ks & 3) + lg) ^ swz_k(lq)) << 3) + (ks >> 2) * 128;
      return *reinterpret_cast<const uint4*>(krow + t4 * 16 * D + pos);
    };
    constexpr int PF = D >= 256 ? 8 : 4;
    constexpr int NR = NS * KSW;  // K fragments of one tile; fragment u: sub-tile u % NS, step u / NS
    uint4 kf[PF + 1];
#pragma unroll
    for (int t4 = 0; t4 < NS; ++t4)
#pragma unroll
      for (int j = 0; j < JT; ++j) sc[j][t4] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < PF; ++u) kf[u] = kfrag(u % NS, u / NS);
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      if (u + PF < NR) kf[(u + PF) % (PF + 1)] = kfrag((u + PF) % NS, (u + PF) / NS);
#pragma unroll
      for (int j = 0; j < JT; ++j)
        sc[j][u % NS] = mfma16x16x32(kf[u % (PF + 1)], qreg[j][u / NS], sc[j][u % NS]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- online softmax (lane: query 16j+lq, keys ts + 16*t4 + 4*lg + i) --------
  // Tiles that lie wholly inside every row's [lo, a] range skip the mask. The
  // probabilities are produced in 32-key steps, one P operand per step.
  auto tile_softmax = [&](Scores& sc, bool need_mask, int ts, uint64_t absent) {
    if (need_mask) {
      // Rows past the tile's last row keep their (zero-query) scores: their
      // outputs are never stored. The empty asm makes the bounds opaque so
      // the compares stay inside this rarely taken branch.
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        int lo_rel = qlo[j] - ts - 4 * lg;
        int hi_rel = qpos[j] - ts - 4 * lg;
        asm volatile("" : "+v"(lo_rel), "+v"(hi_rel));
#pragma unroll
        for (int t4 = 0; t4 < NS; ++t4)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = t4 * 16 + i;
            if (e < lo_rel || e > hi_rel) sc[j][t4][i] = kNegInf;
          }
      }
      if (absent) {
        // Keys of blocks with an invalid table entry are attended by nobody.
        const int b0 = ts >> bs_log2;
#pragma unroll
        for (int t4 = 0; t4 < NS; ++t4)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = ts + t4 * 16 + 4 * lg + i;
            if ((absent >> ((key >> bs_log2) - b0)) & 1u)
#pragma unroll
              for (int j = 0; j < JT; ++j) sc[j][t4][i] = kNegInf;
          }
      }
    }
    // Row maxima in scaled log2 units; chained pairs so each step is one v_max3_f32.
    float mxc[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      float mx = fmaxf(sc[j][0][0], sc[j][0][1]);
#pragma unroll
      for (int e = 2; e < 4 * NS; e += 2)
        mx = fmaxf(fmaxf(mx, sc[j][e >> 2][e & 3]), sc[j][e >> 2][(e & 3) + 1]);
      mxc[j] = max_across_groups(mx) * c;
    }
    // Lazy rescaling: keep the reference max mc[j] until a score exceeds it by
    // more than 2^8 (in log2 units); until then probabilities stay <= 256,
    // harmless in fp32 and bf16, and the final division by the sum taken with
    // the same reference cancels the choice exactly. One vote covers the
    // wave's query tiles, so the common path has no branch between them.
    bool up = false;
#pragma unroll
    for (int j = 0; j < JT; ++j) up = up || mxc[j] > mc[j] + 8.f;
    if (__any(up)) {
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        const float mnew = fmaxf(mc[j], mxc[j]);
        const float alpha = mnew == kNegInf ? 1.f : fast_exp2(mc[j] - mnew);
        mc[j] = mnew;
        negc[j] = mnew == kNegInf ? 0.f : -mnew;
        // Rescale O rows (O layout: lane holds queries 16j + 4*lg + i).
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * lg + i);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[j][nt][i] *= al[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) lsum[j][i] *= al[i];
      }
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        float pr[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[h][i] = fast_exp2(fmaf(sc[j][2 * kk + h][i], c, negc[j]));
        pa[j][kk].x = pack_bf16x2(pr[0][0], pr[0][1]);
        pa[j][kk].y = pack_bf16x2(pr[0][2], pr[0][3]);
        pa[j][kk].z = pack_bf16x2(pr[1][0], pr[1][1]);
        pa[j][kk].w = pack_bf16x2(pr[1][2], pr[1][3]);
      }
    }
  };

  // ---- O += P V ---------------------------------------------------------------
  // B operand of step kk for lane (lq, lg): keys 32kk + 4lg + 0..3 and
  // 32kk + 16 + 4lg + 0..3 (the key set of this lane's P elements) at head_dim
  // column 16nt + lq. ds_read_b64_tr_b16 gives lane j of a 16-lane group
  // element j%4 of the rows addressed by lanes 4k + j/4 (k = 0..3): lane j
  // addresses row key0 + j/4, columns 16nt + 4(j%4) .. +3.
  auto tile_pv = [&](const uint16_t* vs_buf) {
    if constexpr (D >= 256) {
      // The V fragment reads (fragment u: 32-key step u / NTW, column tile
      // u % NTW of the wave's part) run PF fragments ahead of the products, as
      // in tile_s; up to head_dim 128 the compiler's own order measured as
      // fast. A split wave's column tiles start at half * NTW, whole groups of
      // eight: the half only moves the base.
      const int vrow = 4 * lg + (lq >> 2);  // + 32 kk, and + 16: same swizzle
      const uint16_t* vbase = &vs_buf[vrow * D + 4 * (lq & 1)] + half * (NTW / 8) * 128;
      const int vsw = swz_v(vrow);
      auto vfrag = [&](int u) {
        const int kk = u / NTW, nt = u % NTW;
        const int vc = (((2 * (nt & 7) + ((lq & 3) >> 1)) ^ vsw) << 3) + (nt >> 3) * 128 + kk * 32 * D;
        const uint2 v0 = ds_read_tr16(vbase + vc);
        const uint2 v1 = ds_read_tr16(vbase + 16 * D + vc);
        return make_uint4(v0.x, v0.y, v1.x, v1.y);
      };
      constexpr int PF = D >= 256 ? 8 : 4;
      constexpr int NV = NK * NTW;
      uint4 vf[PF + 1];
#pragma unroll
      for (int u = 0; u < PF; ++u) vf[u] = vfrag(u);
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        if (u + PF < NV) vf[(u + PF) % (PF + 1)] = vfrag(u + PF);
        const int kk = u / NTW, nt = u % NTW;
        if (nt == 0) {
#pragma unroll
          for (int j = 0; j < JT; ++j) lsum[j] = mfma16x16x32(pa[j][kk], ones, lsum[j]);
        }
#pragma unroll
        for (int j = 0; j < JT; ++j) o[j][nt] = mfma16x16x32(pa[j][kk], vf[u % (PF + 1)], o[j][nt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
        for (int j = 0; j < JT; ++j) lsum[j] = mfma16x16x32(pa[j][kk], ones, lsum[j]);
        const int vrow = kk * 32 + 4 * lg + (lq >> 2);  // and vrow + 16: same swizzle
        const uint16_t* vbase = &vs_buf[vrow * D + 4 * (lq & 1)];
        const int vsw = swz_v(vrow);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          // Chunk 2nt + b = 16 (nt / 8) + (2 (nt % 8) + b); the swizzle (below 16)
          // touches only the second part.
          const int vc = (((2 * (nt & 7) + ((lq & 3) >> 1)) ^ vsw) << 3) + (nt >> 3) * 128;
          const uint2 v0 = ds_read_tr16(vbase + vc);
          const uint2 v1 = ds_read_tr16(vbase + 16 * D + vc);
          const uint4 vb = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
          for (int j = 0; j < JT; ++j) o[j][nt] = mfma16x16x32(pa[j][kk], vb, o[j][nt]);
        }
      }
    }
  };

  // A tile needs the mask when it reaches past the first row's position or
  // starts before the last row's window start.
  auto needs_mask = [&](int ts) { return (ts + kTileN - 1 > a_min) || (ts < lo_max); };

  // An empty key range (key split only) leaves the row state as it starts:
  // no keys, weight zero in the reduce.
  if (kt_begin <= kt_end) {
    int ent_next = load_entries(kt_begin + 1);
    uint64_t absent_next = stage_load(kt_begin, load_entries(kt_begin), 0);
    stage_store(0);
    __syncthreads();

    // Each tile through all three parts, tile kt+1 streaming into the other
    // buffer meanwhile. The S^T burst runs at raised wave priority, so that a
    // wave issuing back-to-back MFMAs is not held up by the softmax work of the
    // other wave on its SIMD, which fills the gaps.
    Scores sc;
    for (int kt = kt_begin; kt <= kt_end; ++kt) {
      const int buf = (kt - kt_begin) & 1;
      const bool has_next = kt < kt_end;
      const uint64_t absent = absent_next;
      if (has_next) {
        absent_next = stage_load(kt + 1, ent_next, buf ^ 1);
        ent_next = load_entries(kt + 2);
      }
      const int ts = kt * kTileN;
      __builtin_amdgcn_s_setprio(1);
      tile_s(sc, k_s[buf]);
      __builtin_amdgcn_s_setprio(0);
      if constexpr (SPL > 1) {
        // The partner wave (same rows, other half of head_dim) holds the rest
        // of each score: exchange through LDS and add. Both waves add the same
        // two values, so both hold bit-identical scores (and probabilities).
#pragma unroll
        for (int j = 0; j < JT; ++j)
#pragma unroll
          for (int t4 = 0; t4 < NS; ++t4) exch[wave][j * NS + t4][lane] = sc[j][t4];
        __syncthreads();
        const int partner = wave ^ RG;
#pragma unroll
        for (int j = 0; j < JT; ++j)
#pragma unroll
          for (int t4 = 0; t4 < NS; ++t4) {
            const floatx4_t other = exch[partner][j * NS + t4][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[j][t4][i] += other[i];
          }
      }
      tile_softmax(sc, needs_mask(ts) || absent != 0, ts, absent);
      // FP8 codes up to head_dim 128 are widened into the other buffer before
      // the P.V part, so the LDS stores drain under it rather than before the
      // barrier (their loads have landed by then; measured 5% faster, and no
      // faster at head_dim 256 and 512). Direct copies (bf16) only need their
      // wait, as late as possible.
      constexpr bool kEarlyStore = ESZ == 1 && D <= 128;
      if (kEarlyStore && has_next) stage_store(buf ^ 1);
      tile_pv(v_s[buf]);
      if (!kEarlyStore && has_next) stage_store(buf ^ 1);
      __syncthreads();
    }
  }

  if (a.ksplit > 1) {
    // ---- partials of this key range (the reduce normalises) ------------------
#pragma unroll
    for (int j = 0; j < JT; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // Row 16j + 4lg + i's reference max sits in the S^T layout at lane 4lg + i.
        const float m = __shfl(mc[j], 4 * lg + i);
        const int r = r_first + wrow * RPW + 16 * j + 4 * lg + i;
        if (r > r_last) continue;
        const int pos = r / G;
        const int g = r - pos * G;
        const size_t pr = (static_cast<size_t>(ksp) * a.total_q + q0 + pos) * a.hq + kvh * G + g;
        float* acc = a.ws_acc + pr * D;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) acc[(half * NTW + nt) * 16 + lq] = o[j][nt][i] * a.v_scale;
        if (lq == 0 && half == 0) *reinterpret_cast<float2*>(a.ws_ml + pr * 2) = make_float2(m, lsum[j][i]);
      }
    }
    return;
  }

  // ---- normalise and store --------------------------------------------------
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) inv[i] = lsum[j][i] > 0.f ? a.v_scale / lsum[j][i] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r_first + wrow * RPW + 16 * j + 4 * lg + i;
      if (r > r_last) continue;
      const int pos = r / G;
      const int g = r - pos * G;
      uint16_t* orow = a.out + (static_cast<size_t>(q0 + pos) * a.hq + kvh * G + g) * D;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
        orow[(half * NTW + nt) * 16 + lq] = static_cast<uint16_t>(f32_to_bf16_bits(o[j][nt][i] * inv[i]));
    }
  }
}

// Key-split prefill: combine the ksplit partials of each (query token, query
// head). One wave per pair, lane l holding columns l + 64 k; every partial is
// requested before any is used (one round trip), ksplit <= kMaxKeySplit.
constexpr int kMaxKeySplit = 16;

template <int D>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(PrefillParams a) {
  constexpr int CPT = D / 64;
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t pairs = static_cast<size_t>(a.total_q) * a.hq;
  if (pair >= pairs) return;
  const int S = a.ksplit;
  float2 ml[kMaxKeySplit];
  float x[kMaxKeySplit][CPT];
#pragma unroll
  for (int s = 0; s < kMaxKeySplit; ++s) {
    const size_t pr = s * pairs + pair;
    ml[s] = s < S ? *reinterpret_cast<const float2*>(a.ws_ml + pr * 2) : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int k = 0; k < CPT; ++k) x[s][k] = s < S ? a.ws_acc[pr * D + lane + 64 * k] : 0.f;
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxKeySplit; ++s) M = fmaxf(M, ml[s].x);
  float L = 0.f, o[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) o[k] = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxKeySplit; ++s) {
    // A range that saw no key of the row (reference max -inf) weighs zero.
    const float w = ml[s].x == -INFINITY ? 0.f : fast_exp2(ml[s].x - M);
    L = fmaf(ml[s].y, w, L);
#pragma unroll
    for (int k = 0; k < CPT; ++k) o[k] = w != 0.f ? fmaf(x[s][k], w, o[k]) : o[k];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int k = 0; k < CPT; ++k)
    a.out[static_cast<size_t>(pair) * D + lane + 64 * k] = static_cast<uint16_t>(f32_to_bf16_bits(o[k] * inv));
}

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

namespace pagedkv {

// Shared by the bf16 and FP8 entry points and the mixed step; esz: pool
// element bytes (q/out bf16).
int32_t prefill_check(const void* out, const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* cu_q_lens, const int32_t* seq_lens, int32_t batch,
                      int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t num_blocks, float scale, float k_scale, float v_scale,
                      int32_t sliding_window) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
    return fail(PAGED_ERR_INVALID_ARG, "head_dim must be 64, 128, 256 or 512 (got %d)", head_dim);
  if (!pow2_in(block_size, 8, 64))
    return fail(PAGED_ERR_INVALID_ARG, "block_size must be a power of two in [8, 64]");
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads)
    return fail(PAGED_ERR_INVALID_ARG, "need num_q_heads a positive multiple of num_kv_heads");
  if (batch < 0 || total_q < 0 || max_q_len < 0 || max_blocks_per_seq < 1 || num_blocks < 1 ||
      sliding_window < 0)
    return fail(PAGED_ERR_INVALID_ARG, "bad size argument");
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(PAGED_ERR_INVALID_ARG, "scale must be finite and positive");
  if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(PAGED_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if (batch == 0 || total_q == 0 || max_q_len == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !cu_q_lens || !seq_lens)
    return fail(PAGED_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PAGED_ERR_INVALID_ARG, "misaligned pointer");
  // Work items at most: 64 query rows per workgroup (the fewest, at head_dim 512).
  const int64_t items = (static_cast<int64_t>(max_q_len) * (num_q_heads / num_kv_heads) + 63) / 64 *
                        num_kv_heads * batch;
  if (items > (1LL << 30)) return fail(PAGED_ERR_INVALID_ARG, "problem too large");
  return ok();
}

// Query tiles (workgroups without a key split) of a launch.
int64_t prefill_tiles(int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int64_t* per_head) {
  const int group = num_q_heads / num_kv_heads;
  const int tm = kPrefillWaves / splits(head_dim) * rows_per_wave(head_dim);
  *per_head = (static_cast<int64_t>(max_q_len) * group + tm - 1) / tm;
  return *per_head * num_kv_heads;
}

// Key ranges per query tile: 1 when the query tiles alone give every CU a
// workgroup (one resident per CU), else the smallest power of two, at most
// kMaxKeySplit, that does. A function of the shapes and the CU count only.
int prefill_key_splits(int64_t items, int cus) {
  int s = 1;
  while (s < kMaxKeySplit && items * s < cus) s <<= 1;
  return s;
}

size_t prefill_ws_bytes(int ksplit, int32_t total_q, int32_t num_q_heads, int32_t head_dim) {
  return ksplit > 1 ? static_cast<size_t>(ksplit) * total_q * num_q_heads * (head_dim + 2) * sizeof(float) : 0;
}

int32_t prefill_impl(void* out, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* cu_q_lens, const int32_t* seq_lens, int32_t batch,
                     int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, float scale, float k_scale, float v_scale,
                     int32_t sliding_window, void* workspace, size_t workspace_bytes, int esz,
                     void* stream, bool beside_decode) {
  if (int32_t rc = prefill_check(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                                 cu_q_lens, seq_lens, batch, total_q, max_q_len, num_q_heads,
                                 num_kv_heads, head_dim, block_size, num_blocks, scale, k_scale,
                                 v_scale, sliding_window))
    return rc;
  if (workspace && !aligned16(workspace)) return fail(PAGED_ERR_INVALID_ARG, "misaligned workspace");
  if (batch == 0 || total_q == 0 || max_q_len == 0) return ok();
  const int group = num_q_heads / num_kv_heads;
  int64_t tiles = 0;
  const int64_t items1 = prefill_tiles(max_q_len, num_q_heads, num_kv_heads, head_dim, &tiles) * batch;
  int ksplit = 1;
  if (workspace) {
    const int cus = device_cu_count();
    if (cus <= 0) return fail(PAGED_ERR_HIP, "cannot query the device compute-unit count");
    ksplit = prefill_key_splits(items1, cus);
    const size_t need = prefill_ws_bytes(ksplit, total_q, num_q_heads, head_dim);
    if (workspace_bytes < need)
      return fail(PAGED_ERR_INVALID_ARG, "workspace holds %zu bytes, the key split needs %zu", workspace_bytes,
                  need);
  }
  const int64_t items = items1 * ksplit;
  if (items > (1LL << 30)) return fail(PAGED_ERR_INVALID_ARG, "problem too large");
  PrefillParams prm{};
  prm.out = static_cast<uint16_t*>(out);
  prm.q = static_cast<const uint16_t*>(q);
  prm.k_pool = k_pool;
  prm.v_pool = v_pool;
  prm.bt = block_tables;
  prm.cu_q = cu_q_lens;
  prm.seq_lens = seq_lens;
  prm.mb = max_blocks_per_seq;
  prm.hq = num_q_heads;
  prm.hkv = num_kv_heads;
  prm.group = group;
  prm.bs_log2 = ilog2(block_size);
  prm.nb = num_blocks;
  prm.window = sliding_window;
  prm.tiles_per_head = static_cast<int32_t>(tiles);
  prm.ksplit = ksplit;
  prm.work_items = static_cast<int32_t>(items);
  prm.per_xcd = static_cast<int32_t>((items + kNumXcd - 1) / kNumXcd);
  prm.total_q = total_q;
  prm.last_first = beside_decode ? 0 : 1;
  prm.scale_log2 = scale * 1.4426950408889634f * k_scale;
  prm.v_scale = v_scale;
  if (ksplit > 1) {
    prm.ws_acc = static_cast<float*>(workspace);
    prm.ws_ml = prm.ws_acc + static_cast<size_t>(ksplit) * total_q * num_q_heads * head_dim;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(prm.per_xcd * kNumXcd));
  const dim3 block(kPrefillWaves * 64);
  LaunchTrace tr(PAGED_KERNEL_PREFILL, s);
  auto launch = [&](auto kern) {
    hipExtLaunchKernelGGL(kern, grid, block, 0, s, tr.start(), tr.stop(), 0, prm);
  };
  if (head_dim == 512) {
    if (esz == 1) launch(prefill_kernel<512, 1, kPrefillWaves>);
    else launch(prefill_kernel<512, 2, kPrefillWaves>);
  } else if (head_dim == 256) {
    if (esz == 1) launch(prefill_kernel<256, 1, kPrefillWaves>);
    else launch(prefill_kernel<256, 2, kPrefillWaves>);
  } else if (head_dim == 128) {
    if (esz == 1) launch(prefill_kernel<128, 1, kPrefillWaves>);
    else launch(prefill_kernel<128, 2, kPrefillWaves>);
  } else {
    if (esz == 1) launch(prefill_kernel<64, 1, kPrefillWaves>);
    else launch(prefill_kernel<64, 2, kPrefillWaves>);
  }
  tr.finish();
  if (ksplit > 1) {
    const dim3 rgrid(static_cast<unsigned>((static_cast<int64_t>(total_q) * num_q_heads + 3) / 4));
    LaunchTrace rt(PAGED_KERNEL_PREFILL_REDUCE, s);
    auto rlaunch = [&](auto kern) {
      hipExtLaunchKernelGGL(kern, rgrid, dim3(256), 0, s, rt.start(), rt.stop(), 0, prm);
    };
    if (head_dim == 512) rlaunch(prefill_reduce_kernel<512>);
    else if (head_dim == 256) rlaunch(prefill_reduce_kernel<256>);
    else if (head_dim == 128) rlaunch(prefill_reduce_kernel<128>);
    else rlaunch(prefill_reduce_kernel<64>);
    rt.finish();
  }
  return check_launch("paged_attn_prefill_chunk");
}

}  // namespace pagedkv

extern "C" int32_t paged_attn_prefill_chunk(void* out, const void* q, const void* k_pool,
                                            const void* v_pool, const int32_t* block_tables,
                                            int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
                                            const int32_t* seq_lens, int32_t batch,
                                            int32_t total_q, int32_t max_q_len,
                                            int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t block_size,
                                            int32_t num_blocks, float scale,
                                            int32_t sliding_window, void* workspace,
                                            size_t workspace_bytes, int32_t dtype, void* stream) {
  if (dtype != PAGED_BF16)
    return fail(PAGED_ERR_DTYPE, "prefill takes bf16 (FP8 pools: paged_attn_prefill_chunk_fp8)");
  return prefill_impl(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, cu_q_lens,
                      seq_lens, batch, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim,
                      block_size, num_blocks, scale, 1.f, 1.f, sliding_window, workspace,
                      workspace_bytes, 2, stream);
}

extern "C" int32_t paged_attn_prefill_chunk_fp8(void* out, const void* q, const void* k_pool,
                                                const void* v_pool, const int32_t* block_tables,
                                                int32_t max_blocks_per_seq,
                                                const int32_t* cu_q_lens, const int32_t* seq_lens,
                                                int32_t batch, int32_t total_q, int32_t max_q_len,
                                                int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t block_size,
                                                int32_t num_blocks, float scale, float k_scale,
                                                float v_scale, int32_t sliding_window,
                                                void* workspace, size_t workspace_bytes,
                                                void* stream) {
  return prefill_impl(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, cu_q_lens,
                      seq_lens, batch, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim,
                      block_size, num_blocks, scale, k_scale, v_scale, sliding_window, workspace,
                      workspace_bytes, 1, stream);
}

extern "C" int32_t paged_attn_prefill_chunk_workspace_bytes(int32_t batch, int32_t total_q,
                                                            int32_t max_q_len, int32_t num_q_heads,
                                                            int32_t num_kv_heads, int32_t head_dim,
                                                            size_t* bytes) {
  if (!bytes) return fail(PAGED_ERR_INVALID_ARG, "NULL argument");
  *bytes = 0;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
    return fail(PAGED_ERR_INVALID_ARG, "head_dim must be 64, 128, 256 or 512 (got %d)", head_dim);
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads)
    return fail(PAGED_ERR_INVALID_ARG, "need num_q_heads a positive multiple of num_kv_heads");
  if (batch < 0 || total_q < 0 || max_q_len < 0) return fail(PAGED_ERR_INVALID_ARG, "bad size argument");
  if (batch == 0 || total_q == 0 || max_q_len == 0) return ok();
  const int cus = device_cu_count();
  if (cus <= 0) return fail(PAGED_ERR_HIP, "cannot query the device compute-unit count");
  int64_t tiles = 0;
  const int64_t items = prefill_tiles(max_q_len, num_q_heads, num_kv_heads, head_dim, &tiles) * batch;
  *bytes = prefill_ws_bytes(prefill_key_splits(items, cus), total_q, num_q_heads, head_dim);
  return ok();
}
