// prefill_small.hip -- bf16 matrix-core causal GQA prefill for shapes too small to fill
// the chip with one workgroup per q-tile (few heads, short sequences).
//
// Same computation as prefill_mfma.hip: per query head h (K/V head h / G),
// out = softmax(scale * Q K^T + causal mask) V, as the online-softmax recurrence of
// Riftco's "Two exact full-sequence algorithms" over 32-key blocks.  What changes is
// the work split.  With one workgroup per q-tile, a short sequence gives fewer
// workgroups than CUs and the heaviest tile's waves each walk every key alone.  Here a
// workgroup owns one 32-row query slice of one head and splits that slice's keys over
// its waves (2, 4 or 8, by the number of slices): wave w runs the recurrence over its own
// contiguous run of 32-key blocks, and the partial (row max, normalizer, numerator)
// triples are combined exactly in LDS
// at the end, M = max_w m_w, L = sum_w l_w 2^(m_w - M), O = sum_w O_w 2^(m_w - M) / L
// (the same log-sum-exp merge as split-KV decode).  The heaviest slice's critical path
// is then a fraction of its keys, and a short sequence still fills the SIMDs.
//
// Per wave: Q^T fragments in registers for the whole kernel; S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16 with the K fragments loaded straight from global memory in
// the A-operand layout (one block ahead); V rows staged through a wave-private LDS tile
// and read transposed (ds_read_b64_tr_b16) as the A operand of O^T = V^T P^T; lazy
// running max (moved only when a block's max exceeds it by more than 8 in log2 units).
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

constexpr int kBlk = 32;         // keys per block
constexpr float kLazyTau = 8.f;  // log2 growth of the row max tolerated before rescaling

template <int D, int kWaves>
struct SGeo {
  static constexpr int kSteps = D / 16;           // K-steps of the S^T contraction
  static constexpr int kDBlocks = (D + 31) / 32;  // 32-row blocks of O^T
  // V rows are read up to the next multiple of 32 head dims; a stride of 64 or 192
  // mod 256 bytes keeps the transposed reads of four consecutive rows on distinct banks
  static constexpr int kVRead = 64 * kDBlocks;
  static constexpr int kVStride = (kVRead % 256 <= 64) ? kVRead - kVRead % 256 + 64
                                  : (kVRead % 256 <= 192) ? kVRead - kVRead % 256 + 192
                                                          : kVRead - kVRead % 256 + 320;
  static constexpr int kVTile = kBlk * kVStride;         // one wave's V block
  static constexpr int kVLoads = kBlk * D / 8 / 64;      // 16-byte V chunks per lane
  static constexpr int kOStride = D + 4;                 // floats per partial numerator row
  static constexpr int kVBytes = kWaves * kVTile;
  static constexpr int kOBytes = kWaves * 32 * kOStride * 4;
  static constexpr int kSmem = kVBytes > kOBytes ? kVBytes : kOBytes;
};

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int kWaves>
__global__ __launch_bounds__(kWaves * 64, 2) void prefill_small_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ out, int Hq, int Hkv, int T, float c,
    unsigned qsign, int causal, int n_slices, int B, float* __restrict__ lse) {
  using G_ = SGeo<D, kWaves>;
  constexpr int KS = G_::kSteps, DB = G_::kDBlocks, NV = G_::kVLoads;
  // the wave-private V tiles during the key loop, then the partial numerators
  __shared__ __attribute__((aligned(16))) char smem[G_::kSmem];
  __shared__ float part_m[kWaves][32];  // per wave and row: running max (log2 units)
  __shared__ float part_l[kWaves][32];  // and normalizer

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;  // which 16-key half of each 32 the lane holds
  const int col = lane & 31;   // query row of the lane within the slice

  // block -> (slice, head, batch): heaviest slices first
  const int units = Hq * B;
  const int bid = blockIdx.x;
  const int slice = n_slices - 1 - bid / units;
  const int h = (bid % units) % Hq, b = (bid % units) / Hq;
  const int g = h / (Hq / Hkv);
  const int q0 = 32 * slice;
  const int qi = q0 + col;  // the lane's query row (absolute position)

  // keys the slice sees, and this wave's share: an even split of its blocks
  const int kv_end = causal ? min(T, q0 + 32) : T;
  const int nblk = (kv_end + kBlk - 1) / kBlk;
  const int blk0 = wave * nblk / kWaves, blk1 = (wave + 1) * nblk / kWaves;

  const long long kv_base = ((long long)b * Hkv + g) * (long long)T * D;
  const uint16_t* kg = k + kv_base;
  const uint16_t* vg = v + kv_base;

  // Q^T fragments: lane holds query qi, head dims 16*s + 8*half + 0..7
  bf16x8 qf[KS];
  {
    const uint16_t* qrow = q + (((long long)b * Hq + h) * T + qi) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qi < T) x = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * half);
      x ^= qsign;  // negative scale: flip the sign of q exactly, use |scale|
      qf[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  char* vt = smem + wave * G_::kVTile;
  // the padded head dims of the V tile feed discarded numerator rows: keep them finite
  for (int i = lane; i < kBlk * (G_::kVRead - 2 * D) / 16; i += 64) {
    const int per = (G_::kVRead - 2 * D) / 16;
    *reinterpret_cast<u32x4*>(vt + (i / per) * G_::kVStride + 2 * D + (i % per) * 16) = u32x4{0u, 0u, 0u, 0u};
  }

  // K fragments of the block at key j0 (A operand of S^T = K Q^T): key row j0 + col,
  // head dims 16*st + 8*half .. +7; rows past T read row T-1 (those keys are masked)
  auto load_k = [&](int j0, bf16x8 (&kf)[KS]) {
    const uint16_t* kr = kg + (long long)min(j0 + col, T - 1) * D + 8 * half;
#pragma unroll
    for (int st = 0; st < KS; ++st) kf[st] = *reinterpret_cast<const bf16x8*>(kr + 16 * st);
  };
  // V rows of the block, 16-byte chunks: chunk lane + 64*i is row ch / (D/8), chunk ch % (D/8)
  auto load_v = [&](int j0, u32x4 (&vr)[NV]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int ch = lane + 64 * i;
      const int r = ch / (D / 8), cc = ch % (D / 8);
      vr[i] = *reinterpret_cast<const u32x4*>(vg + (long long)min(j0 + r, T - 1) * D + cc * 8);
    }
  };
  auto store_v = [&](const u32x4 (&vr)[NV]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int ch = lane + 64 * i;
      const int r = ch / (D / 8), cc = ch % (D / 8);
      *reinterpret_cast<u32x4*>(vt + r * G_::kVStride + cc * 16) = vr[i];
    }
  };
  // V^T fragments from the wave's tile (transposed reads: inside each 16-lane group,
  // lane s reads 4 head dims (m0 + 4*(s%4) ..) of key row k0p + s/4 and ends up holding
  // head dim m0 + s of keys k0p .. k0p+3)
  auto read_v = [&](bf16x8 (&vf)[2][DB]) {
    const int grp = lane >> 4, sl = lane & 15;
    const int voff = (sl >> 2) * G_::kVStride + (16 * (grp & 1) + 4 * (sl & 3)) * 2;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const char* vrow = vt + (16 * kk + 4 * half) * G_::kVStride + voff;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vrow + db * 64));
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vrow + 8 * G_::kVStride + db * 64));
        vf[kk][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;  // running max, log2 units (same in both lane halves)
  float l_part = 0.f;       // this lane's share of the normalizer
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  bf16x8 kf[KS];
  u32x4 vr[NV];
  if (blk0 < blk1) {
    load_k(kBlk * blk0, kf);
    load_v(kBlk * blk0, vr);
  }
  for (int blk = blk0; blk < blk1; ++blk) {
    const int j0 = kBlk * blk;
    store_v(vr);  // the wave's reads of the previous block were consumed by its products
    bf16x8 kn[KS];
    if (blk + 1 < blk1) {  // next block's loads in flight during this block
      load_k(j0 + kBlk, kn);
      load_v(j0 + kBlk, vr);
    }
    // S^T = K Q^T: accumulator r holds key j0 + 8*(r/4) + 4*half + r%4, this lane's query
    f32x16 s = f32x16{};
#pragma unroll
    for (int st = 0; st < KS; ++st) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], s, 0, 0, 0);
    if ((causal && j0 + kBlk - 1 > q0) || j0 + kBlk > T) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (j >= T || (causal && j > qi)) s[r] = -INFINITY;
      }
    }
    // online softmax, lazy max: every block of a wave holds a key each row sees (key j0
    // is at or before the slice's first row), so m_run is finite from the first block on
    float mx = __builtin_elementwise_maximum(s[0], s[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2)
      mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, s[r]), s[r + 1]);
    mx = pair_max(mx);
    const float mt = mx * c;
    const bool need = mt > m_run + kLazyTau;
    const float m_old = m_run;
    m_run = need ? mt : m_run;
    bf16x8 pb[2];
    float ls[2] = {0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pb[kk][e] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * kk + e], c, -m_run));
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {pb[kk][e], pb[kk][e + 1]};
        ls[kk] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ls[kk], false);
      }
    }
    if (__any(need)) {
      const float alpha = m_old == m_run ? 1.f : __builtin_amdgcn_exp2f(m_old - m_run);
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    l_part += ls[0] + ls[1];
    // O^T += V^T P^T; P's lane order of keys {4h..4h+3, 8+4h..} in each 16-key step is
    // a valid K-ordering because V^T is read in the same order
    bf16x8 vf[2][DB];
    read_v(vf);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kk][db], pb[kk], o[db], 0, 0, 0);
#pragma unroll
    for (int st = 0; st < KS; ++st) kf[st] = kn[st];
  }

  // partial state to LDS (the V tiles' space: every wave is past its key loop first)
  const float l_row = pair_sum(l_part);
  __syncthreads();
  if (half == 0) {
    part_m[wave][col] = m_run;  // -inf with no blocks: weight 0 in the merge
    part_l[wave][col] = l_row;
  }
  float* opart = reinterpret_cast<float*>(smem) + (wave * 32 + col) * G_::kOStride;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int dd = 32 * db + 8 * rq + 4 * half;  // O^T row (head dim) of register 4*rq
      if (dd < D)
        *reinterpret_cast<f32x4*>(opart + dd) =
            f32x4{o[db][4 * rq], o[db][4 * rq + 1], o[db][4 * rq + 2], o[db][4 * rq + 3]};
    }
  __syncthreads();

  // exact merge of the waves' partials: one row and four head dims per item
  for (int it = tid; it < 32 * (D / 4); it += kWaves * 64) {
    const int row = it / (D / 4), d0 = 4 * (it % (D / 4));
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, part_m[w][row]);
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = __builtin_amdgcn_exp2f(part_m[w][row] - M);  // 0 for an empty split
      L += part_l[w][row] * wt;
      acc += *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(smem) +
                                            (w * 32 + row) * G_::kOStride + d0) * wt;
    }
    const int qrow = q0 + row;
    if (qrow < T) {
      const float inv = 1.f / L;
      *reinterpret_cast<f32x4*>(out + (((long long)b * Hq + h) * T + qrow) * D + d0) = acc * inv;
      // row log-sum-exp of the scaled scores, natural log
      if (lse && d0 == 0) lse[((long long)b * Hq + h) * T + qrow] = (M + __log2f(L)) * 0.6931471805599453f;
    }
  }
}

template <int D, int NS>
hipError_t launch_small_ns(const PrefillArgs& a, hipStream_t stream) {
  const int n_slices = (a.T + 31) / 32;
  const long long nblocks = (long long)n_slices * a.Hq * a.B;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  float c = fabsf(a.scale) * 1.4426950408889634f;
  // scale 0: every visible key gets the same weight; a tiny positive factor keeps the
  // masked scores at -inf without changing any visible weight measurably
  if (c == 0.f) c = 1e-30f;
  const unsigned qsign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((prefill_small_kernel<D, NS>), dim3((unsigned)nblocks), dim3(NS * 64), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.out, a.Hq, a.Hkv, a.T, c, qsign, a.causal,
                     n_slices, a.B, a.lse);
  return hipGetLastError();
}

// Key splits per slice: enough waves to cover the SIMDs about two to three times over
// without stretching the heaviest slice's walk (measured at B=4, 12 heads, T=512,
// d=64, 768 slices: 2 splits 10.1 us, 4 splits 11.1 us, 8 splits 15.6 us per launch).
template <int D>
hipError_t launch_small_d(const PrefillArgs& a, hipStream_t stream) {
  const long long slices = (long long)((a.T + 31) / 32) * a.Hq * a.B;
  if (slices <= 320) return launch_small_ns<D, 8>(a, stream);
  if (slices <= 640) return launch_small_ns<D, 4>(a, stream);
  return launch_small_ns<D, 2>(a, stream);
}

}  // namespace

hipError_t launch_attn_prefill_small(const PrefillArgs& a, hipStream_t stream) {
  if (a.window > 0) return hipErrorInvalidValue;  // the local window runs on prefill_mfma
  switch (a.d) {
    case 16: return launch_small_d<16>(a, stream);
    case 32: return launch_small_d<32>(a, stream);
    case 48: return launch_small_d<48>(a, stream);
    case 64: return launch_small_d<64>(a, stream);
    case 80: return launch_small_d<80>(a, stream);
    case 96: return launch_small_d<96>(a, stream);
    case 112: return launch_small_d<112>(a, stream);
    case 128: return launch_small_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
