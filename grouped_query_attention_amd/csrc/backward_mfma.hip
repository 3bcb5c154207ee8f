// backward_mfma.hip -- the memory-linear backward pass of causal GQA attention on bf16
// matrix cores (gfx950).
//
// Riftco's "Two exact full-sequence algorithms": the Flash path keeps only per-row
// softmax statistics from the forward pass; its backward recomputes every probability
// from Q, K and those statistics and applies the exact softmax vector-Jacobian
// product, so no [T, T] buffer exists in either direction.  With s = scale * q.k,
// P_ij = exp(s_ij - lse_i), D_i = sum_d dO_id O_id:
//
//   dV_j = sum_i P_ij dO_i            dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - D_i)        dQ_i = scale sum_j dS_ij k_j
//   dK_j = scale sum_i dS_ij q_i      (K/V gradients summed over the group's heads)
//
// Three kernels, no atomics (results are deterministic):
//  * bwd_prep_kernel: per row, D_i in fp32 from the fp32 dO and O, dO rounded to bf16
//    for the matrix cores, lse converted to log2 units (HBM-bound: 16-byte loads).
//  * bwd_dkdv_kernel: key-parallel.  A wave owns 32 keys of one K/V head (K^T and V^T
//    fragments in registers) and walks the query blocks of every query head of its
//    group.  Scores are formed as S = Q K^T, so each lane holds 16 queries of ONE key:
//    P and dS converted to bf16 are directly the B operands of dV^T += dO^T P and
//    dK^T += Q^T dS, whose A operands come from transposed LDS reads
//    (ds_read_b64_tr_b16) of the row-major Q and dO tiles.
//  * bwd_dq_kernel: query-parallel, the forward kernel's orientation: S^T = K Q^T, each
//    lane one query; dQ^T += K^T dS^T with K^T from transposed reads of the K tile.
// The tiles go from HBM to LDS with direct loads (global_load_lds_dwordx4), two stages
// in two named arrays as in the forward kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct BGeo {
  static constexpr int KS = D / 16;           // K-steps over the head dim
  static constexpr int DB = (D + 31) / 32;    // 32-row blocks of a transposed accumulator
  // Row stride of a tile read both as 16-byte rows and transposed: 64 or 192 mod 256
  // bytes (rows up to the next 32 head dims are read), with which four consecutive rows
  // fall in the four 64-byte quarters of the 256-byte bank window
  static constexpr int kRead = 64 * DB;
  static constexpr int TS = (kRead % 256 <= 64) ? kRead - kRead % 256 + 64
                            : (kRead % 256 <= 192) ? kRead - kRead % 256 + 192
                                                   : kRead - kRead % 256 + 320;
  // row stride read only as 16-byte rows: an odd number of 16-byte chunks
  static constexpr int RS = 2 * D + 16;
};

// Tiles read both ways (TS stride) are swizzled: the 16-byte chunk c of row r is stored
// in chunk slot c ^ ((r >> 2) & 3) of that row.  The 64 banks x 4 bytes of LDS serve a
// ds_read_b128 16 lanes (16 rows of one chunk) at a time and a ds_read_b64_tr_b16 32
// lanes (4 rows x 64 bytes) at a time.  The stride already puts rows r..r+3 in the four
// 64-byte quarters of the bank window, which is what the transposed reads need; the
// swizzle spreads the 16 rows of a row pass over 16 distinct chunks.  TS / 16 is a
// multiple of 4, so a swizzled slot stays inside its row.  (An unpadded 256-byte row
// for d = 128 with a two-level swizzle, conflict-free as well, measured slower.)
__device__ __forceinline__ int swz(int c, int r) { return c ^ ((r >> 2) & 3); }

// Row fragment for MFMA step st of row r (16-byte chunk 2*st + half of the row) in a
// swizzled tile: chunk (2st + half) ^ g with g = (r >> 2) & 3 sits at
// 32*(st ^ (g >> 1)) + 16*(half ^ (g & 1)), i.e. at `even + 32*st` for even st and
// `odd + 32*st` for odd st.
struct SwzRow {
  const char* even;
  const char* odd;
  __device__ __forceinline__ SwzRow(const char* row_start, int r, int half) {
    const int g = (r >> 2) & 3;
    const char* b = row_start + 16 * (half ^ (g & 1));
    even = b + 32 * (g >> 1);
    odd = b - 32 * (g >> 1);
  }
  __device__ __forceinline__ bf16x8 frag(int st) const {
    return *reinterpret_cast<const bf16x8*>((st & 1 ? odd : even) + 32 * st);
  }
};

__device__ __forceinline__ bf16x8 ld_row_frag(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }

// transposed fragment: lane (16-lane group g, slot s) gets head dim m0 + s of the 8 rows
// {4h..4h+3, 8+4h..8+4h+3} + r0 (h = lane / 32) -- the K-ordering of the bf16
// accumulator operands.  `tile` is the first row of the 16-row step (a multiple of 16
// rows into a swizzled tile), `db` the 32-dim block.  The lane's 8 bytes lie in chunk
// 4*db + 2*(g & 1) + ((s >> 1) & 1) of its row.
template <int D>
__device__ __forceinline__ bf16x8 ld_tr_frag(const char* tile, int lane, int db) {
  constexpr int TS = BGeo<D>::TS;
  const int grp = lane >> 4, sl = lane & 15, half = lane >> 5;
  const int c = 4 * db + 2 * (grp & 1) + ((sl >> 1) & 1);
  const int in8 = 8 * (sl & 1);
  const int rlo = 4 * half + (sl >> 2), rhi = rlo + 8;
  const char* lo = tile + rlo * TS + 16 * swz(c, rlo) + in8;
  const char* hi = tile + rhi * TS + 16 * swz(c, rhi) + in8;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)lo);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)hi);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Direct global->LDS loads of a ROWS-row tile of `D` bf16 per row (row i at src + i*2D
// bytes) into LDS rows of STRIDE bytes, swizzled as above when SWZ.  Each wave
// instruction fills 64 consecutive 16-byte slots; slot p is row p / P, chunk slot p % P
// (P = STRIDE / 16), which receives chunk swz(p % P) of its row (padding slots re-read
// chunk 0 and are never used).  A lane's source offset within a tile is the same for
// every tile, so it is computed once per wave instruction.  In a ragged tile, rows at
// or past `valid` re-read row valid-1.
template <int D, int STRIDE, int ROWS, int NW, bool SWZ>
struct TileLoader {
  static constexpr int P = STRIDE / 16, C16 = D / 8, RB = 2 * D;
  static_assert(ROWS * P % 64 == 0, "a tile is a whole number of wave instructions");
  static constexpr int NI = ROWS * P / 64;       // wave instructions per tile
  static constexpr int I = (NI + NW - 1) / NW;   // of which this wave issues at most I
  int off[I];
  int wave_u;
  __device__ __forceinline__ TileLoader(int wave, int lane) {
    wave_u = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int i = 0; i < I; ++i) {
      const int p = (wave + NW * i) * 64 + lane, r = p / P, cc = p % P;
      const int lc = SWZ ? swz(cc, r) : cc;
      off[i] = r * RB + (lc < C16 ? lc : 0) * 16;
    }
  }
  __device__ __forceinline__ void load(const uint16_t* src, char* dst, int valid) const {
    const char* s = reinterpret_cast<const char*>(src);
#pragma unroll
    for (int i = 0; i < I; ++i) {
      const int inst = wave_u + NW * i;
      if (inst < NI) {
        int o = off[i];
        if (valid < ROWS) {
          const int r = o / RB;
          if (r >= valid) o -= (r - valid + 1) * RB;
        }
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(s + o),
                                         (__attribute__((address_space(3))) void*)(dst + inst * 1024), 16, 0, 0);
      }
    }
  }
};

// ---------------------------------------------------------------------------------
// One row per group of 2^lpr_log2 lanes (the power of two at or above d/4), four
// consecutive elements per lane: 16-byte loads of dO and O, an 8-byte store of the bf16
// dO, the row sum reduced over the group.  dO and O are read once: non-temporal loads.
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void bwd_prep_kernel(const float* __restrict__ out, const float* __restrict__ dout,
                                                       const float* __restrict__ lse, uint16_t* __restrict__ dob,
                                                       float* __restrict__ lse2, float* __restrict__ Dv,
                                                       long long rows, int d, int lpr_log2) {
  const int lpr = 1 << lpr_log2;
  const long long row = ((long long)blockIdx.x * 256 + threadIdx.x) >> lpr_log2;
  const int e = 4 * (threadIdx.x & (lpr - 1));
  float acc = 0.f;
  if (row < rows && e < d) {
    const f32x4 g = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dout + row * d + e));
    const f32x4 o = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(out + row * d + e));
    acc = g[0] * o[0] + g[1] * o[1] + g[2] * o[2] + g[3] * o[3];
    const bf16x4 b = {(__bf16)g[0], (__bf16)g[1], (__bf16)g[2], (__bf16)g[3]};
    *reinterpret_cast<bf16x4*>(dob + row * d + e) = b;
  }
  for (int off = lpr >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && e == 0) {
    Dv[row] = acc;
    lse2[row] = lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------------
constexpr int kKvWaves = 4;    // waves per dK/dV workgroup, 32 keys each
constexpr int kKvKeys = 32 * kKvWaves;
constexpr int kQStage = 64;    // query rows per stage of the dK/dV kernel

template <int D>
__global__ __launch_bounds__(kKvWaves * 64, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dob, const float* __restrict__ lse2, const float* __restrict__ Dv,
    float* __restrict__ dk, float* __restrict__ dv, int Hq, int Hkv, int T, float c, float scale, int causal,
    int n_kb) {
  using G = BGeo<D>;
  constexpr int KS = G::KS, DB = G::DB, TS = G::TS;
  constexpr int QS = kQStage;              // query rows per stage
  constexpr int NBLK = QS / 32;            // 32-row blocks per stage
  constexpr int kTile = QS * TS;
  constexpr int kPer = (QS + 63) / 64;  // wave instructions per row statistic
  constexpr int kBuf = 2 * kTile + 2 * kPer * 256;  // Q tile, dO tile, lse2, D
  __shared__ __attribute__((aligned(16))) char lds_a[kBuf];
  __shared__ __attribute__((aligned(16))) char lds_b[kBuf];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  // heaviest key blocks first: under the causal mask the earliest keys see the most
  // queries, so blocks are numbered key block major
  const int nbg = gridDim.x / n_kb;  // batch x K/V heads
  const int bg = blockIdx.x % nbg;
  const int g = bg % Hkv, b = bg / Hkv;
  const int G_ = Hq / Hkv;
  const int k0 = (int)(blockIdx.x / nbg) * kKvKeys;
  const int kw = k0 + 32 * wave;  // this wave's first key
  const int key = kw + col;       // this lane's key (S columns)

  // K^T and V^T fragments of this wave's keys: lane holds key `key`, dims 16*st+8*half..
  bf16x8 kf[KS], vf[KS];
  {
    const long long base = (((long long)b * Hkv + g) * T + key) * D;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
      if (key < T) {
        xk = *reinterpret_cast<const u32x4*>(k + base + 16 * st + 8 * half);
        xv = *reinterpret_cast<const u32x4*>(v + base + 16 * st + 8 * half);
      }
      kf[st] = __builtin_bit_cast(bf16x8, xk);
      vf[st] = __builtin_bit_cast(bf16x8, xv);
    }
  }
  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }

  // query stages: (query head, QS-row block), for every head of the group; causally the
  // rows before the workgroup's first key see none of its keys (k0 is a multiple of QS)
  const int qs0 = causal ? k0 / QS : 0;
  const int nqs = (T + QS - 1) / QS;
  const int per_head = nqs - qs0;
  const int nstages = per_head * G_;
  const TileLoader<D, TS, QS, kKvWaves, true> ld(wave, lane);
  auto stage = [&](int si, char* buf) __attribute__((always_inline)) {
    const int hq = g * G_ + si / per_head;
    const int r0 = (qs0 + si % per_head) * QS;
    const long long rowbase = ((long long)b * Hq + hq) * T + r0;
    const int valid = T - r0;
    ld.load(q + rowbase * D, buf, valid);
    ld.load(dob + rowbase * D, buf + kTile, valid);
    // lse2 and D of the QS rows: kPer wave instructions each (4 bytes per lane)
    if (wave < 2 * kPer) {
      const int part = wave % kPer, r = 64 * part + lane;
      const float* srcf = (wave < kPer ? lse2 : Dv) + rowbase + min(r, valid - 1);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)srcf,
                                       (__attribute__((address_space(3))) void*)(buf + 2 * kTile + wave * 256),
                                       4, 0, 0);
    }
  };

  // S = Q K^T and dP = dO V^T of 32-row block `blk` of a stage: accumulator r holds query
  // row 8*(r/4)+4*half+r%4 of the block, key `key`
  auto sdp = [&](const char* buf, int blk, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
    const SwzRow qrow(buf + (32 * blk + col) * TS, col, half);
    const SwzRow orow(buf + kTile + (32 * blk + col) * TS, col, half);
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qrow.frag(st), kf[st], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(orow.frag(st), vf[st], dp, 0, 0, 0);
    }
    // the row fragments are read kAhead matrix ops ahead of their use (left to itself
    // the scheduler issued each read right before its matrix op, exposing the LDS
    // latency at one wave per SIMD)
    constexpr int kAhead = 2 * KS < 10 ? 2 * KS : 10;
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < 2 * KS - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
  };
  // P = 2^(s*c - lse2) and dS = P (dP - D) in bf16; with `mask`, entries outside the
  // causal triangle or the sequence are exact zeros (first query row of the block: i0)
  auto soft = [&](const char* buf, int blk, const f32x16& s, const f32x16& dp, bf16x8 (&pb)[2], bf16x8 (&sb)[2],
                  bool mask, int i0) __attribute__((always_inline)) {
    const float* l2s = reinterpret_cast<const float*>(buf + 2 * kTile);
    const float* dvs = reinterpret_cast<const float*>(buf + 2 * kTile + kPer * 256);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = 32 * blk + 8 * (r >> 2) + 4 * half + (r & 3);  // row within the stage
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -l2s[qr]));
      if (mask) {
        const int i = i0 + 8 * (r >> 2) + 4 * half + (r & 3);
        const bool ok = i < T && key < T && (!causal || key <= i);
        p = ok ? p : 0.f;
      }
      pb[r >> 3][r & 7] = (__bf16)p;
      sb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dvs[qr]));
    }
  };
  // dV^T += dO^T P and dK^T += Q^T dS over the block's 32 query rows
  auto grad = [&](const char* buf, int blk, const bf16x8 (&pb)[2], const bf16x8 (&sb)[2])
                  __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const char* qt16 = buf + (32 * blk + 16 * kk) * TS;
      const char* ot16 = buf + kTile + (32 * blk + 16 * kk) * TS;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr_frag<D>(ot16, lane, db), pb[kk], dva[db], 0, 0, 0);
        dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr_frag<D>(qt16, lane, db), sb[kk], dka[db], 0, 0, 0);
      }
    }
  };

  // A stage with masks: block by block (a loop, not unrolled: these stages are few),
  // skipping blocks this wave cannot see
  auto compute = [&](int si, const char* buf) __attribute__((always_inline)) {
    const int r0 = (qs0 + si % per_head) * QS;
#pragma unroll 1
    for (int blk = 0; blk < NBLK; ++blk) {
      const int i0 = r0 + 32 * blk;  // first query row of the block
      // causal: rows before this wave's first key see none of its keys
      if (causal && i0 + 31 < kw) continue;
      if (i0 >= T) continue;
      const bool edge = (causal && i0 < kw + 31) || i0 + 32 > T || kw + 32 > T;
      f32x16 s, dp;
      bf16x8 pb[2], sb[2];
      sdp(buf, blk, s, dp);
      soft(buf, blk, s, dp, pb, sb, edge, i0);
      grad(buf, blk, pb, sb);
    }
  };

  // A stage every row and key of which is visible to this wave (no mask): its 32-row
  // blocks as one software pipeline in straight-line code -- block b+1's S and dP
  // products, block b's exp and dS vector work and block b-1's gradient products are
  // independent, so the matrix cores and the vector ALU overlap inside the wave.
  auto compute_fast = [&](const char* buf) __attribute__((always_inline)) {
    f32x16 s[2], dp[2];
    bf16x8 pb[2][2], sb[2][2];
    sdp(buf, 0, s[0], dp[0]);
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      if (blk + 1 < NBLK) sdp(buf, blk + 1, s[(blk + 1) & 1], dp[(blk + 1) & 1]);
      soft(buf, blk, s[blk & 1], dp[blk & 1], pb[blk & 1], sb[blk & 1], false, 0);
      if (blk >= 1) grad(buf, blk - 1, pb[(blk - 1) & 1], sb[(blk - 1) & 1]);
    }
    grad(buf, NBLK - 1, pb[(NBLK - 1) & 1], sb[(NBLK - 1) & 1]);
  };
  // every row of the stage is at or after this wave's last key, inside T, and every key
  // of the wave is inside T
  auto stage_interior = [&](int si) __attribute__((always_inline)) {
    const int r0 = (qs0 + si % per_head) * QS;
    return (!causal || r0 >= kw + 31) && r0 + QS <= T && kw + 32 <= T;
  };
  auto run = [&](int si, const char* buf) __attribute__((always_inline)) {
    if (stage_interior(si))
      compute_fast(buf);
    else
      compute(si, buf);
  };

  if (nstages > 0) {
    stage(0, lds_a);
    if (nstages > 1) stage(1, lds_b);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int si = 0; si < nstages; si += 2) {
      run(si, lds_a);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (si + 2 < nstages) stage(si + 2, lds_a);
      if (si + 1 < nstages) {
        run(si + 1, lds_b);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (si + 3 < nstages) stage(si + 3, lds_b);
      }
    }
  }

  // epilogue: accumulator r of block db holds head dim 32*db + 8*(r/4) + 4*half + r%4
  // of key `key`
  if (key < T) {
    const long long base = (((long long)b * Hkv + g) * T + key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int dd = 32 * db + 8 * rq + 4 * half;
        if (dd < D) {
          f32x4 vk = {dka[db][4 * rq] * scale, dka[db][4 * rq + 1] * scale, dka[db][4 * rq + 2] * scale,
                      dka[db][4 * rq + 3] * scale};
          f32x4 vv = {dva[db][4 * rq], dva[db][4 * rq + 1], dva[db][4 * rq + 2], dva[db][4 * rq + 3]};
          *reinterpret_cast<f32x4*>(dk + base + dd) = vk;
          *reinterpret_cast<f32x4*>(dv + base + dd) = vv;
        }
      }
  }
}

// ---------------------------------------------------------------------------------
constexpr int kQWaves = 8;     // waves per dQ workgroup, 32 query rows each
constexpr int kKStage = 64;    // keys per stage of the dQ kernel

template <int D, int HPW>
__global__ __launch_bounds__(kQWaves * 64, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dob, const float* __restrict__ lse2, const float* __restrict__ Dv,
    float* __restrict__ dq, int Hq, int Hkv, int T, float c, float scale, int causal, int n_qtiles,
    int n_hgroups, int B) {
  using G = BGeo<D>;
  constexpr int KS = G::KS, DB = G::DB, TS = G::TS, RS = G::RS;
  constexpr int SLICES = kQWaves / HPW;
  constexpr int QT = 32 * SLICES;
  constexpr int kKT = kKStage * TS;  // K tile (read as rows and transposed)
  constexpr int kBuf = kKT + kKStage * RS;
  __shared__ __attribute__((aligned(16))) char lds_a[kBuf];
  __shared__ __attribute__((aligned(16))) char lds_b[kBuf];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int per_qt = n_hgroups * B;
  const int bid = blockIdx.x;
  const int qt = n_qtiles - 1 - bid / per_qt;
  const int rem = bid % per_qt;
  const int hg = rem % n_hgroups, b = rem / n_hgroups;
  const int h = hg * HPW + wave / SLICES;
  const int g = (hg * HPW) / (Hq / Hkv);
  const int q0 = qt * QT;
  const int qw = q0 + (wave % SLICES) * 32;
  const int qi = qw + col;

  // Q^T and dO^T fragments (B operands): lane holds query qi, dims 16*st+8*half..
  bf16x8 qf[KS], of[KS];
  const long long qrow = ((long long)b * Hq + h) * T + qi;
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    u32x4 xq = {0u, 0u, 0u, 0u}, xo = {0u, 0u, 0u, 0u};
    if (qi < T) {
      xq = *reinterpret_cast<const u32x4*>(q + qrow * D + 16 * st + 8 * half);
      xo = *reinterpret_cast<const u32x4*>(dob + qrow * D + 16 * st + 8 * half);
    }
    qf[st] = __builtin_bit_cast(bf16x8, xq);
    of[st] = __builtin_bit_cast(bf16x8, xo);
  }
  const float l2 = qi < T ? lse2[qrow] : 0.f;
  const float Dq = qi < T ? Dv[qrow] : 0.f;
  f32x16 dqa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqa[db] = f32x16{};

  const long long kvb = ((long long)b * Hkv + g) * (long long)T;
  const int kend = causal ? min(T, q0 + QT) : T;
  const int nstages = (kend + kKStage - 1) / kKStage;
  const TileLoader<D, TS, kKStage, kQWaves, true> ldk(wave, lane);
  const TileLoader<D, RS, kKStage, kQWaves, false> ldv(wave, lane);
  auto stage = [&](int t, char* buf) __attribute__((always_inline)) {
    const int r0 = t * kKStage;
    ldk.load(k + (kvb + r0) * D, buf, T - r0);
    ldv.load(v + (kvb + r0) * D, buf + kKT, T - r0);
  };
  auto compute = [&](int t, const char* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int blk = 0; blk < kKStage / 32; ++blk) {
      const int j0 = t * kKStage + 32 * blk;
      if ((causal && j0 > qw + 31) || j0 >= T) continue;
      const bool edge = (causal && j0 + 31 > qw) || j0 + 32 > T;
      // S^T = K Q^T and dP^T = V dO^T: accumulator r holds key 8*(r/4)+4*half+r%4 of the
      // block, query qi
      f32x16 s = f32x16{}, dp = f32x16{};
      const SwzRow krow(buf + (32 * blk + col) * TS, col, half);
      const char* vrow = buf + kKT + (32 * blk + col) * RS + half * 16;
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(krow.frag(st), qf[st], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_row_frag(vrow + st * 32), of[st], dp, 0, 0, 0);
      }
      bf16x8 sb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -l2));
        if (edge) {
          const int j = j0 + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool ok = j < T && qi < T && (!causal || j <= qi);
          p = ok ? p : 0.f;
        }
        sb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - Dq));
      }
      // dQ^T += K^T dS^T over the block's 32 keys
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const char* kt16 = buf + (32 * blk + 16 * kk) * TS;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr_frag<D>(kt16, lane, db), sb[kk], dqa[db], 0, 0, 0);
      }
    }
  };

  // A stage all of whose keys are visible to every row of this wave: its 32-key blocks
  // as one software pipeline in straight-line code -- block b+1's S^T and dP^T products,
  // block b's exp and dS vector work and block b-1's dQ products are independent, so the
  // matrix cores and the vector ALU overlap inside the wave.
  auto sdp = [&](const char* buf, int blk, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
    s = f32x16{};
    dp = f32x16{};
    const SwzRow krow(buf + (32 * blk + col) * TS, col, half);
    const char* vrow = buf + kKT + (32 * blk + col) * RS + half * 16;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(krow.frag(st), qf[st], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_row_frag(vrow + st * 32), of[st], dp, 0, 0, 0);
    }
  };
  auto soft = [&](const f32x16& s, const f32x16& dp, bf16x8 (&sb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -l2));
      sb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - Dq));
    }
  };
  auto dqp = [&](const char* buf, int blk, const bf16x8 (&sb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const char* kt16 = buf + (32 * blk + 16 * kk) * TS;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr_frag<D>(kt16, lane, db), sb[kk], dqa[db], 0, 0, 0);
    }
  };
  auto compute_fast = [&](const char* buf) __attribute__((always_inline)) {
    constexpr int NB = kKStage / 32;
    f32x16 s[2], dp[2];
    bf16x8 sb[2][2];
    sdp(buf, 0, s[0], dp[0]);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      if (blk + 1 < NB) sdp(buf, blk + 1, s[(blk + 1) & 1], dp[(blk + 1) & 1]);
      soft(s[blk & 1], dp[blk & 1], sb[blk & 1]);
      if (blk >= 1) dqp(buf, blk - 1, sb[(blk - 1) & 1]);
    }
    dqp(buf, NB - 1, sb[(NB - 1) & 1]);
  };
  auto run = [&](int t, const char* buf) __attribute__((always_inline)) {
    const int j0 = t * kKStage;
    const bool interior = (!causal || j0 + kKStage - 1 <= qw) && j0 + kKStage <= T && qw + 32 <= T;
    if (interior)
      compute_fast(buf);
    else
      compute(t, buf);
  };

  if (nstages > 0) {
    stage(0, lds_a);
    if (nstages > 1) stage(1, lds_b);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < nstages; t += 2) {
      run(t, lds_a);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t + 2 < nstages) stage(t + 2, lds_a);
      if (t + 1 < nstages) {
        run(t + 1, lds_b);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t + 3 < nstages) stage(t + 3, lds_b);
      }
    }
  }

  if (qi < T) {
    float* orow = dq + qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int dd = 32 * db + 8 * rq + 4 * half;
        if (dd < D) {
          f32x4 val = {dqa[db][4 * rq] * scale, dqa[db][4 * rq + 1] * scale, dqa[db][4 * rq + 2] * scale,
                       dqa[db][4 * rq + 3] * scale};
          *reinterpret_cast<f32x4*>(orow + dd) = val;
        }
      }
  }
}

template <int D>
hipError_t launch_d(const BackwardArgs& a, hipStream_t s) {
  const float c = a.scale * kLog2e;
  const int n_kb = (a.T + kKvKeys - 1) / kKvKeys;
  const long long g1 = (long long)a.B * a.Hkv * n_kb;
  if (g1 > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((unsigned)g1), dim3(kKvWaves * 64), 0, s,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.dob, a.lse2, a.Dv, a.dk, a.dv, a.Hq, a.Hkv, a.T, c,
                     a.scale, a.causal, n_kb);
  const int G = a.Hq / a.Hkv;
  const int hpw = G % 2 == 0 ? 2 : 1;
  const int QT = 32 * (kQWaves / hpw);
  const int n_qtiles = (a.T + QT - 1) / QT;
  const int n_hgroups = a.Hq / hpw;
  const long long g2 = (long long)n_qtiles * n_hgroups * a.B;
  if (g2 > 0x7fffffffLL) return hipErrorInvalidValue;
  if (hpw == 2)
    hipLaunchKernelGGL((bwd_dq_kernel<D, 2>), dim3((unsigned)g2), dim3(kQWaves * 64), 0, s,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), a.dob, a.lse2, a.Dv, a.dq, a.Hq, a.Hkv, a.T, c, a.scale,
                       a.causal, n_qtiles, n_hgroups, a.B);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, 1>), dim3((unsigned)g2), dim3(kQWaves * 64), 0, s,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), a.dob, a.lse2, a.Dv, a.dq, a.Hq, a.Hkv, a.T, c, a.scale,
                       a.causal, n_qtiles, n_hgroups, a.B);
  return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(int B, int Hq, int T, int d) {
  const size_t rows = (size_t)B * Hq * T;
  const size_t ob = (rows * d * 2 + 255) / 256 * 256;
  const size_t fb = (rows * 4 + 255) / 256 * 256;
  return ob + 2 * fb;
}

hipError_t launch_attn_backward_mfma(BackwardArgs a, void* workspace, hipStream_t stream) {
  const long long rows = (long long)a.B * a.Hq * a.T;
  char* ws = static_cast<char*>(workspace);
  const size_t ob = ((size_t)rows * a.d * 2 + 255) / 256 * 256;
  const size_t fb = ((size_t)rows * 4 + 255) / 256 * 256;
  a.dob = reinterpret_cast<uint16_t*>(ws);
  a.lse2 = reinterpret_cast<float*>(ws + ob);
  a.Dv = reinterpret_cast<float*>(ws + ob + fb);
  // lanes per row: the power of two at or above d/4 (d is a multiple of 16, at most 128)
  int lpr_log2 = 0;
  while ((1 << lpr_log2) * 4 < a.d) ++lpr_log2;
  const long long pb = ((rows << lpr_log2) + 255) / 256;
  if (pb > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)pb), dim3(256), 0, stream, a.out, a.dout, a.lse,
                     a.dob, a.lse2, a.Dv, rows, a.d, lpr_log2);
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
