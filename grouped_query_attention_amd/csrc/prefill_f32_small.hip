// prefill_f32_small.hip -- fp32 matrix-core causal GQA prefill for shapes too small to
// fill the chip with one workgroup per q-tile (few heads, short sequences).
//
// Same computation as prefill_f32_mfma.hip: per query head h (K/V head h / G),
// out = softmax(scale * Q K^T + causal mask) V with fp32 inputs kept in fp32, the
// products on v_mfma_f32_32x32x2_f32, and the exact online-softmax recurrence of
// Riftco's "Two exact full-sequence algorithms" (running max and normalizer, numerator
// rescaled whenever the max grows).  What changes is the work split, as in
// prefill_small.hip: a workgroup owns one 32-row query slice of one head and splits the
// slice's visible 32-key tiles evenly over its NS waves; each wave runs the recurrence
// over its own contiguous run of tiles, and the NS partial (row max, normalizer,
// numerator) triples are merged exactly in LDS at the end,
// M = max_w m_w, L = sum_w l_w 2^(m_w - M), O = sum_w O_w 2^(m_w - M) / L
// (the log-sum-exp merge of split-KV decode).  A product of the fp32 matrix core takes
// 64 cycles, so one q-tile's keys walked by one wave are a long serial chain; split
// over NS waves that chain shrinks NS-fold and the short sequence fills the SIMDs.
//
// Per wave and 32-key tile (head dims padded with zeros to D, a multiple of 32; lane
// half hh = lane/32 holds head dims hh*D/2 .. of both operands of S^T, so each product
// step sums two head dims D/2 apart):
//   S^T = K Q^T    A = K (key row lane%32), B = Q^T (registers, times scale*log2(e))
//   O^T += V^T P^T  A = V^T (head dim 32*db + lane%32 of key 8*(t/4) + 4*hh + t%4),
//                   B = P^T straight from the score registers (register t of the lane
//                   holds exactly that key).
// Both A operands are loaded from global memory straight into registers, one tile
// ahead: the next tile's K once this tile's S^T products have been issued, its V once
// the P V products have.  No LDS and no barrier inside the key loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.h"

namespace gqa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;  // keys per tile (and query rows per slice)

template <int D, int NS>
struct F32SGeo {
  static constexpr int Half = D / 2;         // head dims per lane half
  static constexpr int DB = D / 32;          // 32-dim blocks of O^T
  static constexpr int OStride = D + 4;      // floats per partial numerator row
};

// combine a value with that of lane l ^ 32 (the other lane half holding the same query):
// swapping the upper half of one copy with the lower half of another leaves the two
// halves' values side by side in every lane
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int NS, bool PAD>
__global__ __launch_bounds__(NS * 64) void prefill_f32_small_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ out, float* __restrict__ lse, int Hq, int Hkv, int T, int d, float scale_log2,
    int causal, int n_slices, int B) {
  using G = F32SGeo<D, NS>;
  constexpr int Half = G::Half, DB = G::DB;
  __shared__ __attribute__((aligned(16))) float opart[NS * 32 * G::OStride];
  __shared__ float part_m[NS][32];  // per wave and row: running max (log2 units)
  __shared__ float part_l[NS][32];  // and normalizer

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;   // lane half
  const int col = lane & 31;  // query row of the lane within the slice (S^T, O^T column)

  // block -> (slice, head, batch): heaviest slices first
  const int units = Hq * B;
  const int bid = blockIdx.x;
  const int slice = n_slices - 1 - bid / units;
  const int h = (bid % units) % Hq, b = (bid % units) / Hq;
  const int g = h / (Hq / Hkv);
  const int q0 = kTile * slice;
  const int qi = q0 + col;  // the lane's query row (absolute position)

  // keys the slice sees, and this wave's share: an even split of its tiles.  Every tile
  // of a causal slice starts at or before the slice's first row, so each row sees a key
  // of every tile it walks and the running max is finite after the first.
  const int kv_end = causal ? min(T, q0 + kTile) : T;
  const int ntile = (kv_end + kTile - 1) / kTile;
  const int t0 = wave * ntile / NS, t1 = (wave + 1) * ntile / NS;

  const long long qbase = ((long long)b * Hq + h) * (long long)T * d;
  const long long kvbase = ((long long)b * Hkv + g) * (long long)T * d;
  const float* kg = k + kvbase;
  const float* vg = v + kvbase;

  // Q^T: head dims hh*Half .. of the lane's row, times scale*log2(e); zero past d or T
  float qf[Half];
  {
    const bool ok = qi < T;
    const float* src = q + qbase + (long long)(ok ? qi : 0) * d + hh * Half;
#pragma unroll
    for (int u = 0; u < Half / 4; ++u) {
      const f32x4 x = (ok && hh * Half + 4 * u < d) ? *reinterpret_cast<const f32x4*>(src + 4 * u)
                                                     : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * u + e] = x[e] * scale_log2;
    }
  }

  // Loads of the next tile are unconditional and of a fixed count, so the wait before a
  // tile's S^T covers its K loads only while its V loads are still in flight.  A head dim
  // past d (PAD) reads an in-row address and is zeroed; a key past T (the ragged last
  // tile only) reads row T-1, which is masked (K) or meets probability 0 (V).  Without
  // padding the row stride is the constant D.
  const int rs = PAD ? d : D;  // floats per K/V row
  // K of the tile at key j0: row j0 + col, head dims hh*Half ..
  float kf[Half];
  auto load_k = [&](int j0, auto ragged_c) {
    constexpr bool kRagged = decltype(ragged_c)::value;
    const int row = kRagged ? min(j0 + col, T - 1) : j0 + col;
    const float* src = kg + (long long)row * rs;
#pragma unroll
    for (int u = 0; u < Half / 4; ++u) {
      const int e0 = hh * Half + 4 * u;
      const bool ok = !PAD || e0 < d;
      f32x4 x = *reinterpret_cast<const f32x4*>(src + (ok ? e0 : 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) kf[4 * u + e] = ok ? x[e] : 0.f;
    }
  };
  // V of the tile at key j0: head dim 32*db + col of key j0 + 8*(t/4) + 4*hh + t%4 in
  // vf[db][t]
  float vf[DB][16];
  auto load_v = [&](int j0, auto ragged_c) {
    constexpr bool kRagged = decltype(ragged_c)::value;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bool ok = !PAD || 32 * db + col < d;
      const float* src = vg + (ok ? 32 * db + col : 0);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int key = j0 + 8 * (t >> 2) + 4 * hh + (t & 3);
        const float x = src[(long long)(kRagged ? min(key, T - 1) : key) * rs];
        vf[db][t] = ok ? x : 0.f;
      }
    }
  };
  auto load_k_at = [&](int j0) {
    if (j0 + kTile > T) load_k(j0, std::true_type{});
    else load_k(j0, std::false_type{});
  };
  auto load_v_at = [&](int j0) {
    if (j0 + kTile > T) load_v(j0, std::true_type{});
    else load_v(j0, std::false_type{});
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = -INFINITY;  // running max of the lane's query (log2 units), same in both halves
  float l = 0.f;        // this lane's share of the normalizer (its 16 keys of every tile)

  if (t0 < t1) {
    load_k_at(kTile * t0);
    load_v_at(kTile * t0);
  }
  for (int t = t0; t < t1; ++t) {
    const int j0 = kTile * t;
    // two accumulation chains: a product that waits on the one just before it leaves
    // the matrix core idle for most of its latency when the SIMD has no other wave
    f32x16 s = f32x16{}, s2 = f32x16{};
#pragma unroll
    for (int i = 0; i < Half; i += 2) {
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[i], qf[i], s, 0, 0, 0);
      s2 = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[i + 1], qf[i + 1], s2, 0, 0, 0);
    }
    s += s2;
    if (t + 1 < t1) load_k_at(j0 + kTile);  // in flight during this tile's softmax and P V

    // mask keys past T and, on the diagonal, keys after the query
    if (j0 + kTile > T || (causal && j0 + kTile - 1 > q0)) {  // wave-uniform
      const int lim = causal ? min(T - 1, qi) : T - 1;  // last key the lane's query sees
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        s[r] = key <= lim ? s[r] : -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = pair_max(mx);
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first tile (m = -inf)
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(s[r] - m);
      l += p[r];
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf[db][r], p[r], o[db], 0, 0, 0);
    if (t + 1 < t1) load_v_at(j0 + kTile);  // in flight during the next tile's S^T and softmax
  }

  // partial state to LDS
  const float l_row = pair_sum(l);
  if (hh == 0) {
    part_m[wave][col] = m;  // -inf with no tiles: weight 0 in the merge
    part_l[wave][col] = l_row;
  }
  float* orow = opart + (wave * 32 + col) * G::OStride;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq)  // O^T row (head dim) of register 4*rq + e
      *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * rq + 4 * hh) =
          f32x4{o[db][4 * rq], o[db][4 * rq + 1], o[db][4 * rq + 2], o[db][4 * rq + 3]};
  __syncthreads();

  // exact merge of the waves' partials: one row and four head dims per item
  for (int it = tid; it < 32 * (D / 4); it += NS * 64) {
    const int row = it / (D / 4), d0 = 4 * (it % (D / 4));
    const int qrow = q0 + row;
    if (qrow >= T || d0 >= d) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NS; ++w) M = fmaxf(M, part_m[w][row]);
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NS; ++w) {
      const float wt = __builtin_amdgcn_exp2f(part_m[w][row] - M);  // 0 for an empty split
      L += part_l[w][row] * wt;
      acc += *reinterpret_cast<const f32x4*>(opart + (w * 32 + row) * G::OStride + d0) * wt;
    }
    const float inv = 1.f / L;
    *reinterpret_cast<f32x4*>(out + qbase + (long long)qrow * d + d0) = acc * inv;
    // row log-sum-exp of the scaled scores, natural log
    if (lse && d0 == 0) lse[((long long)b * Hq + h) * T + qrow] = (M + __log2f(L)) * 0.6931471805599453f;
  }
}

template <int D, int NS>
hipError_t launch_f32_small_ns(const PrefillArgs& a, hipStream_t stream) {
  const int n_slices = (a.T + kTile - 1) / kTile;
  const long long nblocks = (long long)n_slices * a.Hq * a.B;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  auto kern = a.d == D ? prefill_f32_small_kernel<D, NS, false> : prefill_f32_small_kernel<D, NS, true>;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblocks), dim3(NS * 64), 0, stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), a.out, a.lse, a.Hq, a.Hkv, a.T, a.d,
                     a.scale * 1.4426950408889634f, a.causal, n_slices, a.B);
  return hipGetLastError();
}

// Key splits per slice, by the number of slices (at D > 64 at most 4: eight partial
// numerators of 32 x D floats would leave room for one workgroup per CU).
template <int D>
hipError_t launch_f32_small_d(const PrefillArgs& a, hipStream_t stream) {
  const long long slices = (long long)((a.T + kTile - 1) / kTile) * a.Hq * a.B;
  if constexpr (D <= 64) {
    if (slices <= 320) return launch_f32_small_ns<D, 8>(a, stream);
  }
  if (slices <= 640) return launch_f32_small_ns<D, 4>(a, stream);
  return launch_f32_small_ns<D, 2>(a, stream);
}

}  // namespace

hipError_t launch_attn_prefill_f32_small(const PrefillArgs& a, hipStream_t stream) {
  if (a.window > 0) return hipErrorInvalidValue;  // the local window runs on prefill_f32_mfma
  switch ((a.d + 31) / 32) {  // d a multiple of 16, padded to the next multiple of 32
    case 1: return launch_f32_small_d<32>(a, stream);
    case 2: return launch_f32_small_d<64>(a, stream);
    case 3: return launch_f32_small_d<96>(a, stream);
    case 4: return launch_f32_small_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
