// decode_mfma.hip -- split-KV cached GQA decode for gfx950 (bf16 cache, fp32 out).
//
// The new tokens at positions startPos .. startPos+n-1 attend to every cached key up
// to their own position (makarna's CausalAttentionCached key limit startPos+qi+1).
// Every call reads the whole visible cache once -- the cost the multi-query primer's
// section 2.4 "Incremental: one token at a time" points at -- so the kernel is built
// to stream K and V at HBM rate:
//
//  * Work item = one wave = (sequence b, K/V head g, key chunk).  The G*n query rows of
//    the group (G query heads x n tokens) are the columns of one 16-wide MFMA tile, so
//    every K/V byte is read once per group, not once per query head.
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: the A operand (16 keys x 32 head
//    dims) is loaded straight from HBM -- each load instruction reads 16 key rows x
//    64 contiguous bytes -- and Q^T stays in registers.
//  * O^T = V^T P^T needs V with keys along the contraction; the 32-key V tile goes
//    through a wave-private LDS tile and ds_read_b64_tr_b16.  The S^T accumulator,
//    converted to bf16, is the P^T operand directly (keys in the order
//    {4g..4g+3, 16+4g..16+4g+3} for lane group g; V^T uses the same order).
//  * The next tile's K and V are in flight while the current one is computed.
//  * Online softmax in log2 units with a lazily moved running max.  Each chunk leaves
//    a partial (m, l, O) in the workspace; decode_merge_kernel combines them:
//    M = max m_s, L = sum l_s 2^(m_s - M), O = sum O_s 2^(m_s - M) / L.
//    The merge is exact in exact arithmetic; it is the per-row statistics of Riftco's
//    "Two exact full-sequence algorithms" applied across key chunks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace gqa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 4;        // independent waves per workgroup
constexpr int kTile = 32;        // keys per tile
constexpr int kCols = 16;        // query columns per MFMA tile
constexpr float kLazyTau = 8.f;  // log2 growth of the running max tolerated before rescale
// Split target: two waves per SIMD (256 CUs x 4 SIMDs).  Every wave of a launch walks a
// chunk of the same length, so a wave count that is not a whole multiple of the SIMD
// count leaves a partial last round (1536 waves for the 64 x 8 KV heads of a 32768-key
// history ran at 5.8 TB/s, 2048 at 7.0).  Longer chunks also mean fewer partials to merge:
// 8192 waves ran at 6.6 TB/s, 4096 at 6.9.
constexpr int kSimds = 1024;
constexpr int kTargetWaves = 2 * kSimds;

template <int D>
struct DGeo {
  static constexpr int kSteps = (D + 31) / 32;  // 32-wide K-steps of S^T (last may be padded)
  static constexpr int kDBlocks = D / 16;       // 16-row blocks of O^T
  static constexpr int kChunks = kTile * D / 8;  // 16-byte chunks of a V tile
  static constexpr int kPerLane = kChunks / 64;  // V chunks staged per lane
  // Transposed reads of the 4 lane groups touch 16 consecutive rows x 32 bytes; an odd
  // multiple of 32 bytes as row stride spreads each half-wave over 8 distinct 32-byte
  // bank slots.
  static constexpr int kVStride = ((2 * D / 32) % 2 == 1) ? 2 * D : 2 * D + 32;
  static constexpr int kLdsPerWave = kTile * kVStride;
};

// Where the K/V history lives: one contiguous [B, Hkv, L, d] cache, or a pool of blocks
// addressed through a per-sequence block table.  A block is head-major [Hkv, bs, d]
// (rstride d, hstride bs*d) or token-major [bs, Hkv, d] (rstride Hkv*d, hstride d); its
// rows are 2*d contiguous bytes either way.
struct KvSource {
  const uint16_t* k;
  const uint16_t* v;
  const int* table;  // paged: [B, max_blocks] physical block of each logical block
  const int* lens;   // paged: [B] history length of each sequence (new tokens included)
  int L;             // contiguous: rows per head in the cache
  int start_pos;     // contiguous: position of the first new token (every sequence)
  int bs, max_blocks, num_blocks, max_len;  // paged
  int window;        // local window (keys p-W+1 .. p); 0 = none
  int rstride;                 // paged: elements from one position to the next of a head
  long long hstride, bstride;  // paged: elements from one K/V head to the next; per block
  int head_fast;  // 1: consecutive waves take the K/V heads of one (sequence, chunk)
};

// First key the kernels walk: the first new token's window start, rounded down to the
// 32-key tile (so 16-row groups stay inside 16-aligned blocks); 0 without a window.
__host__ __device__ __forceinline__ int key_begin(int kv_len, int n, int window) {
  if (window <= 0) return 0;
  const int lo = kv_len - n - window + 1;
  return lo <= 0 ? 0 : (lo / kTile) * kTile;
}

__device__ __forceinline__ float xmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// reduce over the 4 lane groups (lanes l, l^16, l^32, l^48 hold the same query column)
__device__ __forceinline__ float group_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = xmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
  return xmax(x, __shfl_xor(x, 16));
}
__device__ __forceinline__ float group_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  return x + __shfl_xor(x, 16);
}

template <int D, bool PAGED>
__global__ __launch_bounds__(kWaves * 64, 2) void decode_split_kernel(
    const uint16_t* __restrict__ q, const KvSource kv, float* __restrict__ opart,
    float* __restrict__ mlpart, int n, int Hq, int Hkv, float c, int nsplit, int chunk, int ncb,
    int total_waves) {
  using G_ = DGeo<D>;
  __shared__ __attribute__((aligned(16))) char smem[kWaves * G_::kLdsPerWave];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gw = blockIdx.x * kWaves + wave;
  if (gw >= total_waves) return;  // whole wave; no workgroup barrier is used
  // wave -> (sequence b, K/V head g, column block cb, chunk split).  With token-major
  // blocks the K/V heads of a position share its rows, so their waves go side by side.
  int split, cb, g, b;
  if (kv.head_fast) {
    g = gw % Hkv;
    const int r = gw / Hkv;
    split = r % nsplit;
    cb = (r / nsplit) % ncb;
    b = r / nsplit / ncb;
  } else {
    split = gw % nsplit;
    const int unit = gw / nsplit;
    cb = unit % ncb;
    g = unit / ncb % Hkv;
    b = unit / ncb / Hkv;
  }
  const int G = Hq / Hkv;
  const int ncols = G * n;
  int kv_len;  // keys any new token can see: the sequence's history length
  if constexpr (PAGED) {
    kv_len = kv.lens[b];
    if (kv_len < n || kv_len > kv.max_len) return;  // the merge marks the sequence's rows
  } else {
    kv_len = kv.start_pos + n;
  }
  const int start_pos = kv_len - n;
  const int last = kv_len - 1;  // rows past it are never read
  const int kbeg = key_begin(kv_len, n, kv.window);
  const int c0 = kbeg + split * chunk;
  if (c0 >= kv_len) return;  // empty chunk: the merge only reads chunks below kv_len
  const int c1 = min(c0 + chunk, kv_len);

  const int col = lane & 15;  // query column of the lane
  const int grp = lane >> 4;  // lane group: keys 4*grp.. of each 16-key block
  const int cidx = cb * kCols + col;
  const bool col_ok = cidx < ncols;
  const int tok = col_ok ? cidx / G : 0;  // columns are token-major: (token, head in group)
  const int hq = g * G + (col_ok ? cidx % G : 0);
  const int qpos = start_pos + tok;  // absolute position of the column's token
  const int qlo = kv.window > 0 ? qpos - kv.window + 1 : 0;  // its first visible key

  // Q^T fragments: column cidx, head dims 32*st + 8*grp + 0..7 (zero past D)
  bf16x8 qf[G_::kSteps];
#pragma unroll
  for (int st = 0; st < G_::kSteps; ++st) {
    const int d0 = 32 * st + 8 * grp;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (col_ok && d0 < D)
      x = *reinterpret_cast<const u32x4*>(q + (((long long)b * n + tok) * Hq + hq) * D + d0);
    qf[st] = __builtin_bit_cast(bf16x8, x);
  }

  // Where a 32-key tile's rows live.  A tile is two 16-row groups; group kb covers rows
  // j0+16kb .. j0+16kb+15, clamped to `last`.  Rows of one group are evenly spaced in
  // memory (rs elements apart): in the contiguous cache trivially, in a pool because a
  // block holds a multiple of 16 positions.  rows[kb] is the element offset of the
  // group's first (clamped) row; row r of the group is at
  // rows[kb] + (min(j0+16kb+r, last) - first)*rs.
  const long long head_base = ((long long)b * Hkv + g) * (long long)kv.L * D;  // contiguous
  const int rs = PAGED ? kv.rstride : D;
  const int* tab = PAGED ? kv.table + (long long)b * kv.max_blocks : nullptr;
  bool bad = false;  // a table entry outside the pool: the sequence's rows become NaN
  // table entries of a tile's two groups; fetched one tile ahead of the K/V loads with
  // vector loads (a scalar load would share its wait counter with the LDS traffic)
  auto fetch = [&](int j0, int (&e)[2]) {
    if constexpr (PAGED) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        int blk = min(j0 + 16 * kb, last) / kv.bs;
        asm volatile("" : "+v"(blk));  // keep the address per lane: a vector load
        e[kb] = tab[blk];
      }
    }
  };
  auto resolve = [&](int j0, const int (&e)[2], long long (&rows)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int first = min(j0 + 16 * kb, last);
      if constexpr (PAGED) {
        int ent = __builtin_amdgcn_readfirstlane(e[kb]);
        if (ent < 0 || ent >= kv.num_blocks) {
          bad = true;
          ent = 0;
        }
        rows[kb] = (long long)ent * kv.bstride + (long long)g * kv.hstride +
                   (long long)(first % kv.bs) * kv.rstride;
      } else {
        rows[kb] = head_base + (long long)first * D;
      }
    }
  };
  char* vl = smem + wave * G_::kLdsPerWave;

  // K fragments of a tile (A operand): block kb, step st -> key j0 + 16kb + col,
  // head dims 32st + 8grp .. +7.  The cache is streamed once per call, so K and V are
  // read with non-temporal loads (they stream at 7.0 TB/s on this part, plain loads of
  // the same pattern at 6.2 TB/s).
  auto load_k = [&](int j0, const long long (&rows)[2], bf16x8 (&kf)[2][G_::kSteps]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int first = min(j0 + 16 * kb, last);
      const long long row = rows[kb] + (long long)(min(j0 + 16 * kb + col, last) - first) * rs;
#pragma unroll
      for (int st = 0; st < G_::kSteps; ++st) {
        const int d0 = 32 * st + 8 * grp;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (d0 < D) x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kv.k + row + d0));
        kf[kb][st] = __builtin_bit_cast(bf16x8, x);
      }
    }
  };
  // V tile rows j0..j0+31, contiguous 16-byte chunks per lane (4 rows per 1 KB load)
  auto load_v = [&](int j0, const long long (&rows)[2], u32x4 (&vr)[G_::kPerLane]) {
#pragma unroll
    for (int i = 0; i < G_::kPerLane; ++i) {
      const int ch = lane + 64 * i;
      const int r = ch / (D / 8), cc = ch % (D / 8);
      const int kb = r >> 4;
      const int first = min(j0 + 16 * kb, last);
      const long long row = (kb ? rows[1] : rows[0]) + (long long)(min(j0 + r, last) - first) * rs;
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kv.v + row + cc * 8));
    }
  };
  auto store_v = [&](const u32x4 (&vr)[G_::kPerLane]) {
#pragma unroll
    for (int i = 0; i < G_::kPerLane; ++i) {
      const int ch = lane + 64 * i;
      const int r = ch / (D / 8), cc = ch % (D / 8);
      *reinterpret_cast<u32x4*>(vl + r * G_::kVStride + cc * 16) = vr[i];
    }
  };

  f32x4 o[G_::kDBlocks];
#pragma unroll
  for (int db = 0; db < G_::kDBlocks; ++db) o[db] = f32x4{};
  float m_run = -INFINITY, l_part = 0.f;

  // transposed-read addressing: lane s of group grp reads 4 head dims (16db + 4(s%4) ..)
  // of key row k0 + s/4; after the transpose it holds head dim 16db + s of keys k0..k0+3
  const int sl = lane & 15;
  const int voff = (sl >> 2) * G_::kVStride + 4 * (sl & 3) * 2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  bf16x8 kf[2][G_::kSteps];
  u32x4 vr[G_::kPerLane];
  int ent[2] = {0, 0}, ent_next[2] = {0, 0};
  long long rows[2];
  fetch(c0, ent);
  resolve(c0, ent, rows);
  load_k(c0, rows, kf);
  load_v(c0, rows, vr);
  if (c0 + kTile < c1) fetch(c0 + kTile, ent_next);
  for (int j0 = c0; j0 < c1; j0 += kTile) {
    store_v(vr);  // this wave's earlier reads of the tile buffer are complete
    bf16x8 kn[2][G_::kSteps];
    const bool more = j0 + kTile < c1;
    if (more) {
      resolve(j0 + kTile, ent_next, rows);
      load_k(j0 + kTile, rows, kn);
      load_v(j0 + kTile, rows, vr);
      if (j0 + 2 * kTile < c1) fetch(j0 + 2 * kTile, ent_next);
    }

    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int st = 0; st < G_::kSteps; ++st)
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][st], qf[st], s[kb], 0, 0, 0);
    }
    // keys past the chunk, after the column's own position, or below its window get
    // no weight
    if (j0 + kTile > c1 || j0 + kTile - 1 > start_pos || (kv.window > 0 && j0 < kv_len - kv.window)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + 16 * kb + 4 * grp + r;
          if (j >= c1 || j > qpos || j < qlo) s[kb][r] = -INFINITY;
        }
    }
    float mx = xmax(xmax(xmax(s[0][0], s[0][1]), xmax(s[0][2], s[0][3])),
                    xmax(xmax(s[1][0], s[1][1]), xmax(s[1][2], s[1][3])));
    mx = group_max(mx);
    const float mt = mx * c;
    const bool need = mt > m_run + kLazyTau;
    if (__any(need)) {
      const float m_new = need ? mt : m_run;
      // lanes that keep their max keep their scale: exp2(m - m) would be NaN
      // for a column that has seen only masked keys (m = -inf)
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < G_::kDBlocks; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    // a column whose keys so far are all masked keeps m = -inf: use 0 as reference
    const float m_ref = m_run == -INFINITY ? 0.f : m_run;
    bf16x8 pb;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        pb[4 * kb + r] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -m_ref));
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 pr = {pb[e], pb[e + 1]};
      l_part = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_part, false);
    }

    // O^T += V^T P^T over the tile's 32 keys (one K-step)
    const char* v0 = vl + (4 * grp) * G_::kVStride + voff;
#pragma unroll
    for (int db = 0; db < G_::kDBlocks; ++db) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + db * 32));
      const i16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + 16 * G_::kVStride + db * 32));
      const bf16x8 a =
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[db], 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < G_::kSteps; ++st) kf[kb][st] = kn[kb][st];
    }
  }

  // partial (m, l, O) of this chunk for every valid column.  O^T row (head dim) of
  // accumulator r in block db is 16db + 4grp + r.  A bad table entry poisons the
  // chunk (m = l = NaN), and the merge carries the NaN into every row of the group.
  float l_tot = group_sum(l_part);
  if (bad) {
    m_run = __builtin_nanf("");
    l_tot = __builtin_nanf("");
  }
  if (col_ok) {
    const long long pidx = ((long long)(b * Hkv + g) * nsplit + split) * ncols + cidx;
    float* op = opart + pidx * D;
#pragma unroll
    for (int db = 0; db < G_::kDBlocks; ++db)
      *reinterpret_cast<f32x4*>(op + 16 * db + 4 * grp) = o[db];
    if (grp == 0) {
      mlpart[2 * pidx] = m_run;
      mlpart[2 * pidx + 1] = l_tot;
    }
  }
}

// One 64-thread block per output row (b, g, column): combine the chunk partials.
template <int D, bool PAGED>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ opart,
                                                          const float* __restrict__ mlpart,
                                                          float* __restrict__ out, const KvSource kv,
                                                          int n, int Hq, int Hkv, int nsplit,
                                                          int chunk) {
  constexpr int PER = (D + 63) / 64;
  const int G = Hq / Hkv;
  const int ncols = G * n;
  const int row = blockIdx.x;  // (b * Hkv + g) * ncols + cidx
  const int cidx = row % ncols;
  const int bg = row / ncols;
  const int g = bg % Hkv, b = bg / Hkv;
  const int tok = cidx / G, hq = g * G + cidx % G;
  float* orow = out + (((long long)b * n + tok) * Hq + hq) * D;
  int kv_len;
  if constexpr (PAGED) {
    kv_len = kv.lens[b];
    if (kv_len < n || kv_len > kv.max_len) {  // no valid history: the row is NaN
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int d = threadIdx.x + 64 * e;
        if (d < D) orow[d] = __builtin_nanf("");
      }
      return;
    }
  } else {
    kv_len = kv.start_pos + n;
  }
  const int nvalid = (kv_len - key_begin(kv_len, n, kv.window) + chunk - 1) / chunk;
  const long long base = (long long)bg * nsplit * ncols + cidx;  // partial index of split 0

  float M = -INFINITY;
  for (int s = 0; s < nvalid; ++s) M = xmax(M, mlpart[2 * (base + (long long)s * ncols)]);
  float Lsum = 0.f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int s = 0; s < nvalid; ++s) {
    const long long p = base + (long long)s * ncols;
    const float w = __builtin_amdgcn_exp2f(mlpart[2 * p] - M);  // 0 for an all-masked chunk
    Lsum += mlpart[2 * p + 1] * w;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int d = threadIdx.x + 64 * e;
      if (d < D) acc[e] += opart[p * D + d] * w;
    }
  }
  const float inv = 1.f / Lsum;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int d = threadIdx.x + 64 * e;
    if (d < D) orow[d] = acc[e] * inv;
  }
}

template <int D, bool PAGED>
hipError_t launch_d(const DecodeArgs& a, const KvSource& kv, const DecodePlan& p,
                    hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int ncols = G * a.n;
  const int ncb = (ncols + kCols - 1) / kCols;
  const long long total = (long long)a.B * a.Hkv * ncb * p.nsplit;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  const long long np = (long long)a.B * a.Hkv * p.nsplit * ncols;
  float* opart = static_cast<float*>(a.workspace);
  float* mlpart = opart + np * D;
  const float c = a.scale * 1.4426950408889634f;
  const int blocks = (int)((total + kWaves - 1) / kWaves);
  hipLaunchKernelGGL((decode_split_kernel<D, PAGED>), dim3(blocks), dim3(kWaves * 64), 0, stream,
                     static_cast<const uint16_t*>(a.q), kv, opart, mlpart, a.n, a.Hq, a.Hkv, c,
                     p.nsplit, p.chunk, ncb, (int)total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D, PAGED>), dim3(a.B * a.Hkv * ncols), dim3(64), 0,
                     stream, opart, mlpart, a.out, kv, a.n, a.Hq, a.Hkv, p.nsplit, p.chunk);
  return hipGetLastError();
}

template <bool PAGED>
hipError_t launch_any_d(const DecodeArgs& a, const KvSource& kv, const DecodePlan& p,
                        hipStream_t stream) {
  switch (a.d) {
    case 16: return launch_d<16, PAGED>(a, kv, p, stream);
    case 32: return launch_d<32, PAGED>(a, kv, p, stream);
    case 48: return launch_d<48, PAGED>(a, kv, p, stream);
    case 64: return launch_d<64, PAGED>(a, kv, p, stream);
    case 80: return launch_d<80, PAGED>(a, kv, p, stream);
    case 96: return launch_d<96, PAGED>(a, kv, p, stream);
    case 112: return launch_d<112, PAGED>(a, kv, p, stream);
    case 128: return launch_d<128, PAGED>(a, kv, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int decode_key_span(int len, int n, int window) {
  if (window <= 0) return len;
  // the widest case: key_begin rounds the window start down by up to kTile - 1 keys
  const long long span = (long long)window + n - 1 + (kTile - 1);
  return span < len ? (int)span : len;
}

// Share of the SIMDs busy over the rounds a launch of `waves` equal waves needs
static double simd_fill(long long waves) {
  const long long rounds = (waves + kSimds - 1) / kSimds;
  return (double)waves / (double)(rounds * kSimds);
}

// Pure function of the shape: enough chunks that the launch has at least ~kTargetWaves
// waves, preferring (among up to twice that many chunks) the smallest count whose waves
// fill the SIMDs evenly; each chunk a multiple of the 32-key tile; partials are (d + 2)
// floats per chunk, query row and head.  `total_len` is the most keys one sequence walks.
DecodePlan plan_decode(int B, int n, int total_len, int Hq, int Hkv, int d, int dtype) {
  DecodePlan p{1, total_len, 0, false};
  p.mfma = dtype == kBF16 && d % 16 == 0 && d <= 128 && total_len > 0;
  if (!p.mfma) return p;
  const int ncols = (Hq / Hkv) * n;
  const long long units = (long long)B * Hkv * ((ncols + kCols - 1) / kCols);
  long long want = (kTargetWaves + units - 1) / units;
  const long long max_split = (total_len + kTile - 1) / kTile;
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  // chunks are whole tiles, so the split asked for and the split made can differ
  auto chunk_for = [&](long long w) { return ((total_len + w - 1) / w + kTile - 1) / kTile * kTile; };
  auto split_for = [&](long long w) { return (total_len + chunk_for(w) - 1) / chunk_for(w); };
  if (units * split_for(want) >= kSimds / 2) {
    long long best = want;
    double fill = simd_fill(units * split_for(want));
    for (long long w = want + 1; w <= 2 * want && w <= max_split && fill < 0.9; ++w) {
      const double f = simd_fill(units * split_for(w));
      if (f > fill + 0.05) {
        best = w;
        fill = f;
      }
    }
    want = best;
  }
  const long long chunk = chunk_for(want);
  p.chunk = (int)chunk;
  p.nsplit = (int)((total_len + chunk - 1) / chunk);
  p.workspace = (size_t)B * Hq * n * (size_t)p.nsplit * (size_t)(d + 2) * sizeof(float);
  return p;
}

hipError_t launch_attn_decode_mfma(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  KvSource kv{static_cast<const uint16_t*>(a.kc), static_cast<const uint16_t*>(a.vc), nullptr,
              nullptr, a.L, a.start_pos, 0, 0, 0, 0, a.window, a.d, 0, 0, 0};
  return launch_any_d<false>(a, kv, p, stream);
}

hipError_t launch_attn_decode_paged(const DecodeArgs& a, const PagedArgs& pg, const DecodePlan& p,
                                    hipStream_t stream) {
  KvSource kv{static_cast<const uint16_t*>(a.kc), static_cast<const uint16_t*>(a.vc), pg.table,
              pg.seq_lens, 0, 0, pg.block_size, pg.max_blocks, pg.num_blocks,
              pg.block_size * pg.max_blocks, a.window, 0, 0, 0, 0};
  const long long d = a.d, bs = pg.block_size, blk = (long long)a.Hkv * bs * d;
  if (pg.token_major) {  // [num_blocks, bs, Hkv, d]
    kv.rstride = a.Hkv * a.d;
    kv.hstride = d;
    kv.head_fast = 1;
  } else {  // [num_blocks, Hkv, bs, d]
    kv.rstride = a.d;
    kv.hstride = bs * d;
  }
  kv.bstride = blk;
  return launch_any_d<true>(a, kv, p, stream);
}

}  // namespace gqa
