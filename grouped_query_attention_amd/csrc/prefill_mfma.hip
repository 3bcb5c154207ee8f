// prefill_mfma.hip -- bf16 matrix-core causal GQA prefill for gfx950.
//
// Computes, per query head h (K/V head g = h / G), out = softmax(scale * Q K^T + mask) V
// with the causal mask of Hesper's "Causal Masking" section, as the memory-linear
// online-softmax algorithm of Riftco's "Two exact full-sequence algorithms": running
// row max and normalizer, numerator rescaled as key tiles arrive, no [T, T] buffer.
//
// Mapping onto CDNA4:
//  * A workgroup of 8 waves owns one q-tile of 256/HPW query rows for HPW query heads
//    of the same K/V group (HPW = 2 when the group has an even number of heads), each
//    wave 32 rows of one head.  Each K/V tile is staged once in LDS and read by
//    every wave: the GQA reuse of "Grouped-Query Attention" section 5.1 lands
//    in LDS, not in a repeat_interleave copy.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    A = K rows straight from LDS, B = Q^T held in registers for the whole kernel.
//    In the 32x32 accumulator every lane then holds 16 keys of ONE query, so row
//    reductions are in-lane plus one permlane32 swap between the two lane halves.
//  * The same accumulator, converted to bf16, is the B operand of O^T = V^T P^T: its
//    lane holds keys {4h..4h+3, 8+4h..8+4h+3} (h = lane/32) of each 16-key step,
//    which is a valid K-ordering as long as the A operand (V^T) uses the same one.
//    ds_read_b64_tr_b16 reads four consecutive keys of one head-dim column out of the
//    row-major V tile, so V never needs a transposed copy.
//  * Online softmax in log2 units over 32-key blocks (scale*log2(e) folded into one
//    FMA before v_exp_f32); the running max is only moved when a block's max exceeds it
//    by more than 8, so the O rescale is skipped on almost every block (p stays below
//    2^8).
//  * K/V rows go from HBM straight into LDS (global_load_lds_dwordx4, no register
//    staging) in stages of 128 keys, double-buffered in two separate LDS arrays; stage
//    t+1's loads are in flight during all of stage t.
//  * A stage fully visible to every row of a wave runs as a software pipeline over its
//    four blocks: the softmax of block b (vector ALU) beside the S^T of block b+1 and
//    the P V of block b-1 (matrix core), interleaved by sched_group_barrier.
//  * Causal skipping: 32-key blocks entirely above a wave's diagonal are not computed;
//    the mask is only evaluated in diagonal stages.  A local window (the multi-query
//    primer's local attention, section 4.1: keys p-W+1 .. p) skips from both sides:
//    stages below the workgroup's first window start are never loaded, blocks below a
//    wave's window are not computed, and window-edge blocks are masked.
//  * Dispatch order: (batch, head group) units in chunks sized so that one round of
//    resident workgroups covers every q-tile of a chunk, heaviest q-tiles first inside
//    a chunk; blocks of one unit keep the same block-id residue mod 8, i.e. stay on one
//    XCD and share its L2.
//  * Head dims that are 16 mod 32 (the P V product runs over the next multiple of 32):
//    the first padded V column in LDS holds ones, so the normalizer accumulates in the
//    numerator's row D on the matrix core instead of in vector sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.h"

namespace gqa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWgWaves = 8;     // waves per workgroup (HPW heads x kWgWaves/HPW row slices)
constexpr int kBN = 64;         // keys per compute tile
constexpr int kSub = 2;         // compute tiles per LDS stage (one barrier per stage)
constexpr int kStage = kSub * kBN;
constexpr float kLazyTau = 8.f; // log2 growth of the row max tolerated before rescaling

template <int D>
struct Geo {
  static constexpr int kSteps = D / 16;           // K-steps of the S^T contraction
  static constexpr int kDBlocks = (D + 31) / 32;  // 32-row blocks of O^T
  // K rows: an odd number of 16-byte chunks apart, so the 16 lanes served per bank
  // cycle (same column, 16 consecutive rows) hit 16 different 16-byte bank groups.
  static constexpr int kKStride = 2 * D + 16;
  // V rows: per bank cycle (64 banks x 4 bytes) the transposed reads of 32 lanes touch
  // 4 consecutive rows x 64 bytes; a row stride of 64 or 192 mod 256 bytes puts those
  // 4 rows in distinct banks (measured conflict-free; 32 mod 128 is not).  Rows are
  // read up to the next multiple of 32 head dims; the padding feeds discarded O^T rows,
  // except that for head dims 16 mod 32 its first column holds ones (the normalizer).
  static constexpr int kVRead = 64 * kDBlocks;
  static constexpr int kVStride = (kVRead % 256 <= 64) ? kVRead - kVRead % 256 + 64
                                  : (kVRead % 256 <= 192) ? kVRead - kVRead % 256 + 192
                                                          : kVRead - kVRead % 256 + 320;
  static constexpr int kKTile = kStage * kKStride;
  static constexpr int kVTile = kStage * kVStride;
  static constexpr int kBuf = kKTile + kVTile;  // one stage: K tile then V tile
};

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int HPW, bool WIN>
__global__ __launch_bounds__(kWgWaves * 64, 2) void prefill_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ out, int Hq, int Hkv, int T, float c,
    unsigned qsign, int causal, int window_arg, int n_qtiles, int n_hgroups, int B,
    float* __restrict__ lse, int chunk_units) {
  using G_ = Geo<D>;
  // Head dims 16 mod 32: the P V product runs over the next multiple of 32, and the
  // first padded V column holds ones, so the numerator's row D accumulates the
  // normalizer (with every rescale applied to it as to the numerator).
  constexpr bool kOnesCol = D % 32 == 16;
  // the local window is a separate instantiation: plain causal attention carries none
  // of its checks
  const int window = WIN ? window_arg : 0;
  constexpr int SLICES = kWgWaves / HPW;  // 32-row slices per head
  constexpr int QT = 32 * SLICES;         // query rows per head per workgroup
  // Two stages in two separate LDS arrays: the loop is unrolled by two so each
  // iteration reads one array while direct global->LDS loads fill the other, and the
  // compiler can see they do not alias (one shared array indexed by the stage makes it
  // wait for the in-flight loads before every LDS read).
  __shared__ __attribute__((aligned(16))) char lds_a[G_::kBuf];
  __shared__ __attribute__((aligned(16))) char lds_b[G_::kBuf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;   // which 16-key half of each 32 the lane holds
  const int col = lane & 31;    // query column of the lane in its wave's 32 rows

  // block -> (q-tile, head group, batch).  Units (batch, head group) are taken in
  // chunks of chunk_units, every q-tile of a chunk before the next chunk, heaviest
  // q-tiles first inside a chunk: the workgroups in flight then cover all q-tiles of a
  // few units, whose K/V stay in L2 (blocks of a unit share their residue mod 8 when
  // chunk_units is a multiple of 8, so they run on one XCD).
  const int units = n_hgroups * B;
  const int bid = blockIdx.x;
  const int chunk = bid / (chunk_units * n_qtiles);
  const int in_chunk = min(chunk_units, units - chunk * chunk_units);
  const int bid_in = bid - chunk * chunk_units * n_qtiles;
  const int qt = n_qtiles - 1 - bid_in / in_chunk;
  const int rem = chunk * chunk_units + bid_in % in_chunk;
  const int hg = rem % n_hgroups;
  const int b = rem / n_hgroups;
  const int h = hg * HPW + wave / SLICES;
  const int g = (hg * HPW) / (Hq / Hkv);
  const int q0 = qt * QT;
  const int qw = q0 + (wave % SLICES) * 32;   // first query row of this wave
  const int qi = qw + col;               // this lane's query row (absolute position)

  const long long kv_base = ((long long)b * Hkv + g) * (long long)T * D;
  const uint16_t* kg = k + kv_base;
  const uint16_t* vg = v + kv_base;

  // Q^T fragments: lane holds query qi, head dims 16*s + 8*half + 0..7
  bf16x8 qf[G_::kSteps];
  {
    const uint16_t* qrow = q + (((long long)b * Hq + h) * T + qi) * D;
#pragma unroll
    for (int s = 0; s < G_::kSteps; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qi < T) x = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * half);
      x ^= qsign;  // negative scale: flip the sign of q exactly, use |scale|
      qf[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 o[G_::kDBlocks];
#pragma unroll
  for (int db = 0; db < G_::kDBlocks; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;  // running max, log2 units (same in both lane halves)
  float l_part = 0.f;       // this lane's share of the normalizer

  const int kend = causal ? min(T, q0 + QT) : T;
  const int nstages = (kend + kStage - 1) / kStage;
  // a local window (causal only) also drops the stages below the first row's window
  const int t0 = window > 0 ? max(0, q0 - window + 1) / kStage : 0;

  // Tile staging with direct global->LDS loads (global_load_lds_dwordx4, no register
  // staging): one wave instruction writes 64 consecutive 16-byte LDS slots; slot p of a
  // tile is row p / P, chunk p % P of a row padded to P chunks.  A lane's source offset
  // inside a tile is the same for every tile, so it is computed once here, as one byte
  // offset per wave instruction.  Padding slots re-read chunk 0 of their row.  In a
  // ragged last tile, rows at or past T read row T-1 instead: those keys are masked,
  // and their finite values meet probability 0.
  constexpr int KP = G_::kKStride / 16, VP = G_::kVStride / 16, C16 = D / 8, RB = D * 2;
  constexpr int KI = (kSub * KP + kWgWaves - 1) / kWgWaves;  // wave instructions per wave per stage
  constexpr int VI = (kSub * VP + kWgWaves - 1) / kWgWaves;
  unsigned koff[KI], voff[VI];
  bool vpad[VI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int p = (wave + kWgWaves * i) * 64 + lane, cc = p % KP;
    koff[i] = (p / KP) * RB + (cc < C16 ? cc : 0) * 16;
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int p = (wave + kWgWaves * i) * 64 + lane, cc = p % VP;
    voff[i] = (p / VP) * RB + (cc < C16 ? cc : 0) * 16;
    vpad[i] = cc >= C16;
  }
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // clamp a source offset to the last valid row of a ragged stage
  auto clamp_row = [&](unsigned off, int rmax) -> unsigned {
    const int r = (int)(off / RB);
    return r > rmax ? off - (unsigned)((r - rmax) * RB) : off;
  };
  // One stage's loads.  A stage inside T issues every load from the stage's base (an
  // SGPR pair) plus the lane's fixed 32-bit offset, with no vector arithmetic; only a
  // ragged last stage clamps its rows.
  auto issue = [&](const char* kb, const char* vb, char* dst, int rmax, auto ragged_c) {
    constexpr bool kRagged = decltype(ragged_c)::value;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int inst = wave_u + kWgWaves * i;
      if (inst < kSub * KP) {
        const unsigned off = kRagged ? clamp_row(koff[i], rmax) : koff[i];
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(kb + off),
            (__attribute__((address_space(3))) void*)(dst + inst * 1024), 16, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int inst = wave_u + kWgWaves * i;
      if (inst < kSub * VP && !(kOnesCol && vpad[i])) {
        const unsigned off = kRagged ? clamp_row(voff[i], rmax) : voff[i];
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(vb + off),
            (__attribute__((address_space(3))) void*)(dst + G_::kKTile + inst * 1024), 16, 0, 0);
      }
    }
  };
  auto stage = [&](int t, char* dst) {
    const char* kb = reinterpret_cast<const char*>(kg) + (long long)t * kStage * RB;
    const char* vb = reinterpret_cast<const char*>(vg) + (long long)t * kStage * RB;
    // (the window instantiation keeps one load path: a second copy costs it registers)
    if (WIN || t * kStage + kStage > T)
      issue(kb, vb, dst, T - 1 - t * kStage, std::true_type{});
    else
      issue(kb, vb, dst, 0, std::false_type{});
  };

  // ---- per-block pieces.  The online softmax runs over 32-key blocks: a block's S^T
  // is one 32x32 accumulator in which every lane holds 16 keys of its own query.
  constexpr int KS = G_::kSteps, DB = G_::kDBlocks;
  constexpr int kBlk = 32;                // keys per softmax block
  constexpr int kNB = kStage / kBlk;      // blocks per LDS stage

  // K fragments of the block whose first K row is kl: the lane holds key row `col`,
  // head dims 16*st + 8*half .. +7 (the A operand of S^T = K Q^T)
  auto read_k = [&](const char* kl, bf16x8 (&kf)[KS]) {
    const char* krow = kl + col * G_::kKStride + half * 16;
#pragma unroll
    for (int st = 0; st < KS; ++st) kf[st] = *reinterpret_cast<const bf16x8*>(krow + st * 32);
  };
  // V^T fragments of the block whose first V row is vl.  Transposed-read addressing
  // inside each 16-lane group: lane s reads 4 head dims (m0 + 4*(s%4) ..) of key row
  // (k0p + s/4); after the transpose lane s holds head dim m0 + s of keys k0p .. k0p+3.
  auto read_v = [&](const char* vl, bf16x8 (&vf)[2][DB]) {
    const int grp = lane >> 4, sl = lane & 15;
    const int voff = (sl >> 2) * G_::kVStride + (16 * (grp & 1) + 4 * (sl & 3)) * 2;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const char* vrow = vl + (16 * kk + 4 * half) * G_::kVStride + voff;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vrow + db * 64));
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vrow + 8 * G_::kVStride + db * 64));
        vf[kk][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  // S^T = K Q^T for one block: accumulator r holds key 8*(r/4) + 4*half + r%4 of the
  // block, for this lane's query
  auto mfma_s = [&](const bf16x8 (&kf)[KS], f32x16& s) {
    s = f32x16{};
#pragma unroll
    for (int st = 0; st < KS; ++st) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], s, 0, 0, 0);
  };
  // O^T += V^T P^T over one block; P's lane order of keys {4h..4h+3, 8+4h..} in each
  // 16-key step is a valid K-ordering because V^T is read in the same order
  auto mfma_pv = [&](const bf16x8 (&vf)[2][DB], const bf16x8 (&pb)[2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kk][db], pb[kk], o[db], 0, 0, 0);
  };
  // mask of a diagonal or window-edge block at key k0
  auto mask_blk = [&](f32x16& s, int k0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
      const bool ok = causal ? (j <= qi && (window <= 0 || j > qi - window)) : (j < T);
      if (!ok) s[r] = -INFINITY;
    }
  };
  // Online-softmax step for one block: move the running max lazily (only when it grows
  // by more than kLazyTau), rescale the normalizer, and form p = 2^(s*c - m) in bf16.
  // Returns whether any lane moved its max; the numerator must then be scaled by
  // `alpha` before this block's P V is added.
  auto softmax_blk = [&](const f32x16& s, bf16x8 (&pb)[2], float& m_old, float& lsum) -> bool {
    // NaN-propagating maximum lowers to v_maximum3_f32 with no operand
    // canonicalization (fmaxf would add one v_max per score)
    float mx = __builtin_elementwise_maximum(s[0], s[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2)
      mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, s[r]), s[r + 1]);
    mx = pair_max(mx);
    const float mt = mx * c;  // block max in log2 units
    const bool need = mt > m_run + kLazyTau;
    m_old = m_run;
    m_run = need ? mt : m_run;
    // p, rounded to bf16 for the P V product.  Under a window a column can meet a
    // block entirely below its window before any visible key (m = -inf): 0 is then the
    // reference, and its p are exact zeros.
    const float m_ref = (WIN && m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pb[kk][e] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * kk + e], c, -m_ref));
    if constexpr (!kOnesCol) {
      // the normalizer sums the same bf16 values, two per v_dot2_f32_bf16 against (1, 1)
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      float ls[2] = {0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {pb[kk][e], pb[kk][e + 1]};
          ls[kk] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ls[kk], false);
        }
      lsum = ls[0] + ls[1];
    }
    return __any(need);
  };
  // A block moved the max of some columns (rare with the lazy threshold): scale the
  // numerator by 2^(m_old - m_new) and return the factor, by which the caller scales
  // the normalizer of the earlier blocks before adding this block's sum.  Columns that
  // kept their max keep their scale (2^(m - m) would be NaN for a column that has seen
  // only masked keys, m = -inf).
  auto rescale_o = [&](float m_old) {
    const float alpha = m_old == m_run ? 1.f : __builtin_amdgcn_exp2f(m_old - m_run);
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    return alpha;
  };

  // P V of an interior stage's last block, deferred past the stage barrier (its V
  // fragments are already in registers) so it runs beside the next stage's first S^T.
  bf16x8 pend_v[2][DB];
  bf16x8 pend_p[2];
  bool pending = false;

  // Stage whose blocks are all fully visible to every row of this wave: a software
  // pipeline over its blocks.  Region b runs the softmax of block b on the vector ALU
  // beside the S^T of block b+1 and the P V of block b-1 on the matrix core, so the
  // wave's own instruction stream keeps both busy.
  auto interior_stage = [&](const char* kl, const char* vl, int k0s, auto masked) {
    constexpr bool kMasked = decltype(masked)::value;
    f32x16 s[kNB];
    bf16x8 pb[kNB][2];
    {
      bf16x8 kf[KS];
      read_k(kl, kf);
      if (pending) mfma_pv(pend_v, pend_p);  // needs no LDS: covers the K read latency
      mfma_s(kf, s[0]);
    }
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      bf16x8 kf[KS];
      bf16x8 vf[2][DB];
      if (b + 1 < kNB) read_k(kl + (b + 1) * kBlk * G_::kKStride, kf);
      if (b >= 1) read_v(vl + (b - 1) * kBlk * G_::kVStride, vf);
      float m_old, lsum = 0.f;
      if constexpr (kMasked) mask_blk(s[b], k0s + b * kBlk);
      const bool resc = softmax_blk(s[b], pb[b], m_old, lsum);
      if (b + 1 < kNB) mfma_s(kf, s[b + 1]);
      if (b >= 1) mfma_pv(vf, pb[b - 1]);
      // interleave: K reads, the max (vector ops), then one matrix op per four vector
      // ops; the V reads go out once the first S^T ops have freed their K registers
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        if (i >= 3 && i < 11) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      if (resc) {  // after P V of block b-1, before that of block b
        const float a = rescale_o(m_old);
        if constexpr (!kOnesCol) l_part *= a;
      }
      if constexpr (!kOnesCol) l_part += lsum;
    }
    read_v(vl + (kNB - 1) * kBlk * G_::kVStride, pend_v);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) pend_p[kk] = pb[kNB - 1][kk];
    pending = true;
  };

  // Any other stage (a diagonal with blocks the wave does not see, a window edge, a
  // ragged end): block by block, with the visibility and mask checks.
  auto edge_stage = [&](int t, const char* kl, const char* vl) {
    if (pending) {
      mfma_pv(pend_v, pend_p);
      pending = false;
    }
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const int k0 = t * kStage + b * kBlk;
      // keys k0.. are all beyond this wave's last row, past T, or below the window of
      // its first row: nothing to do.  The mask is needed where some key is after
      // the first row or below the last row's window.
      const bool active = (!causal || k0 <= qw + 31) && k0 < T &&
                          (window <= 0 || k0 + kBlk - 1 > qw - window);
      if (!active) continue;
      const bool diag = causal ? (k0 + kBlk - 1 > qw || (window > 0 && k0 <= qw + 31 - window))
                               : (k0 + kBlk > T);
      bf16x8 kf[KS];
      read_k(kl + b * kBlk * G_::kKStride, kf);
      f32x16 s;
      mfma_s(kf, s);
      if (diag) mask_blk(s, k0);
      bf16x8 pb[2];
      float m_old, lsum = 0.f;
      if (softmax_blk(s, pb, m_old, lsum)) {
        const float a = rescale_o(m_old);
        if constexpr (!kOnesCol) l_part *= a;
      }
      if constexpr (!kOnesCol) l_part += lsum;
      bf16x8 vf[2][DB];
      read_v(vl + b * kBlk * G_::kVStride, vf);
      mfma_pv(vf, pb);
    }
  };

  // Stages alternate between the two LDS arrays.  Stage t+1's loads are in flight
  // while stage t is computed; right after the barrier that ends stage t (every wave
  // has read it) stage t+2's loads go into the array stage t held.
  auto step = [&](int t, char* cur) {
    const int ks = t * kStage;
    bool inter = ks + kStage <= T;
    if (causal) inter = inter && ks + kStage - 1 <= qw;               // below the diagonal
    if (WIN && window > 0) inter = inter && ks > qw + 31 - window;    // inside every window
    // A causal diagonal stage every block of which holds a key this wave's rows see runs
    // the pipeline too, with the mask applied to each block's scores: a block no row of
    // a column sees gives exact zeros (the column's running max is already finite), and
    // the pipeline costs less than skipping the few invisible blocks saves.  (With a
    // window the masked pipeline measured slower; those stages keep the edge path.)
    const bool all_active = !WIN && causal && ks + kStage <= T && ks + kStage - kBlk <= qw + 31;
    if (inter)
      interior_stage(cur, cur + G_::kKTile, ks, std::false_type{});
    else if (all_active)
      interior_stage(cur, cur + G_::kKTile, ks, std::true_type{});
    else
      edge_stage(t, cur, cur + G_::kKTile);
    __builtin_amdgcn_s_waitcnt(0);  // stage t+1 has landed in LDS
    __syncthreads();
    if (t + 2 < nstages) stage(t + 2, cur);
  };

  if constexpr (kOnesCol) {
    // the padded V chunks read by the P V product: (1, 0, ..., 0) then zeros, in every
    // row of both stage arrays; the stage loads never write them
    constexpr int kPadChunks = G_::kVRead / 16 - C16;
    for (int i = tid; i < 2 * kStage * kPadChunks; i += kWgWaves * 64) {
      const int arr = i / (kStage * kPadChunks), rem = i % (kStage * kPadChunks);
      const int row = rem / kPadChunks, ch = rem % kPadChunks;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (ch == 0) val[0] = 0x3f80u;  // bf16 1.0 in the low half: head dim D
      char* base = (arr == 0 ? lds_a : lds_b) + G_::kKTile + row * G_::kVStride + (C16 + ch) * 16;
      *reinterpret_cast<u32x4*>(base) = val;
    }
  }
  // the first stage alone before the first barrier: at launch every workgroup's first
  // loads come from HBM at once, and the second stage is in flight during the first's
  // compute either way
  stage(t0, lds_a);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t0 + 1 < nstages) stage(t0 + 1, lds_b);
  for (int t = t0; t < nstages; t += 2) {
    step(t, lds_a);
    if (t + 1 < nstages) step(t + 1, lds_b);
  }
  if (pending) mfma_pv(pend_v, pend_p);
  // epilogue: O^T row (head dim) of accumulator r in block db is
  // 32*db + 8*(r/4) + 4*half + r%4; column is this lane's query.
  // accumulator r = 8 of the last block holds head dim 32*(DB-1) + 16 = D in the lanes
  // of half 0 (the ones column) and D + 4 (a zero column) in half 1
  const float l_row = pair_sum(kOnesCol ? o[DB - 1][8] : l_part);
  const float inv = 1.f / l_row;
  // row log-sum-exp of the scaled scores, natural log: (m + log2 l) * ln 2 (m is the
  // reference the p were taken against, in log2 units)
  if (lse && qi < T && half == 0)
    lse[((long long)b * Hq + h) * T + qi] = (m_run + __log2f(l_row)) * 0.6931471805599453f;
  if (qi < T) {
    float* orow = out + (((long long)b * Hq + h) * T + qi) * D;
#pragma unroll
    for (int db = 0; db < G_::kDBlocks; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int dd = 32 * db + 8 * rq + 4 * half;
        if (dd < D) {
          f32x4 val = {o[db][4 * rq] * inv, o[db][4 * rq + 1] * inv, o[db][4 * rq + 2] * inv,
                       o[db][4 * rq + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + dd) = val;
        }
      }
  }
}

// Units per chunk of the dispatch order: about one round of resident workgroups (one
// per CU) covers every q-tile of a chunk's units; at least 32 units, a multiple of 8.
int chunk_units(int n_qtiles, int units) {
  int c = 256 / n_qtiles / 8 * 8;
  if (c < 32) c = 32;
  return c < units ? c : units;
}

template <int D, int HPW, bool WIN>
hipError_t launch_dh(const PrefillArgs& a, hipStream_t stream) {
  constexpr int QT = 32 * (kWgWaves / HPW);
  const int n_qtiles = (a.T + QT - 1) / QT;
  const int n_hgroups = a.Hq / HPW;
  const long long nblocks = (long long)n_qtiles * n_hgroups * a.B;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  float c = fabsf(a.scale) * 1.4426950408889634f;
  // scale 0: every visible key gets the same weight; a tiny positive factor keeps the
  // masked scores at -inf without changing any visible weight measurably
  if (c == 0.f) c = 1e-30f;
  const unsigned qsign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((prefill_mfma_kernel<D, HPW, WIN>), dim3((unsigned)nblocks), dim3(kWgWaves * 64), 0,
                     stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.out, a.Hq, a.Hkv, a.T, c, qsign, a.causal,
                     a.causal ? a.window : 0, n_qtiles, n_hgroups, a.B, a.lse,
                     chunk_units(n_qtiles, n_hgroups * a.B));
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const bool win = a.causal && a.window > 0;
  if (G % 2 == 0) return win ? launch_dh<D, 2, true>(a, stream) : launch_dh<D, 2, false>(a, stream);
  return win ? launch_dh<D, 1, true>(a, stream) : launch_dh<D, 1, false>(a, stream);
}

}  // namespace

long long prefill_mfma_grid(int B, int Hq, int Hkv, int T) {
  const int hpw = (Hq / Hkv) % 2 == 0 ? 2 : 1;
  const int qt = 32 * (kWgWaves / hpw);
  return (long long)((T + qt - 1) / qt) * (Hq / hpw) * B;
}

bool prefill_mfma_supported(int dtype, int d, int Hq, int Hkv) {
  return dtype == kBF16 && d > 0 && d <= 128 && d % 16 == 0 && Hkv > 0 && Hq % Hkv == 0;
}

hipError_t launch_attn_prefill_mfma(const PrefillArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 16: return launch_d<16>(a, stream);
    case 32: return launch_d<32>(a, stream);
    case 48: return launch_d<48>(a, stream);
    case 64: return launch_d<64>(a, stream);
    case 80: return launch_d<80>(a, stream);
    case 96: return launch_d<96>(a, stream);
    case 112: return launch_d<112>(a, stream);
    case 128: return launch_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
