// prefill_f32_mfma.hip -- fp32 causal GQA prefill on the fp32 matrix cores.  Head dims are
// multiples of 16 up to 128; the kernel works on d rounded up to 32, with zero padding.
//
// With a local window W (the multi-query primer's local attention, section 4.1) row i
// sees keys i-W+1 .. i only: the stage loop starts at the workgroup's first window
// start, a wave skips tiles wholly below its rows' windows, and tiles that cross a
// window edge are masked like diagonal tiles.
//
// Same computation as the other prefill kernels (scores = scale * Q K^T, causal mask,
// softmax over keys, times V; query head h reads K/V head h / (Hq/Hkv)), with fp32
// inputs kept in fp32: the products run on v_mfma_f32_32x32x2_f32, which multiplies
// and accumulates in fp32.  The online softmax (running max and normalizer, numerator
// rescaled when the max grows) is the exact recurrence of Riftco's "Two exact
// full-sequence algorithms"; it equals the materialized softmax up to rounding.
//
// Work split: a workgroup owns 128 query rows of one query head (two heads of one K/V
// group at d = 128 when the group size is even), one wave
// per 32 rows.  Key tiles of 32 keys are staged through LDS: K row-major, V transposed,
// each loaded from HBM into registers one tile ahead.
//
// Per wave and tile:
//   S^T = K Q^T   A = K (32 keys x 2 head dims per step, from LDS), B = Q^T (registers).
//                 Lane l owns query l%32 and, in its 16 accumulator registers, keys
//                 8*(r/4) + 4*(l/32) + r%4: the row max is an in-lane max plus one swap
//                 with lane l^32.  Lane half h = l/32 holds head dims h*D/2 .. of both
//                 operands, so each step sums two head dims D/2 apart.
//   O^T += V^T P^T  A = V^T (32 head dims x 2 keys, from the transposed LDS tile),
//                 B = P^T straight from the score registers: step t takes key
//                 8*(t/4) + 4*(l/32) + t%4, which is exactly register t of the lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace gqa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;                    // waves per query head (128 rows)
constexpr int kRows = 32;                    // query rows per wave
constexpr int kKeys = 32;                    // keys per tile
constexpr int kVtStride = kKeys + 4;         // floats per V^T row: 9 16-byte chunks (odd)

template <int D, int HPW>
struct F32Geo {
  static constexpr int Threads = kWaves * 64 * HPW;
  static constexpr int KStride = D + 4;      // floats per K row: an odd number of 16-byte chunks
  static constexpr int Half = D / 2;         // head dims per lane half
  static constexpr int DB = D / 32;          // 32-dim blocks of O^T
  static constexpr int C4 = D / 4;           // 16-byte chunks per row
  static constexpr int LPT = kKeys * C4 / Threads;  // chunks per thread per tensor and tile
  static_assert(D % 32 == 0 && LPT * Threads == kKeys * C4, "a tile must split evenly over the threads");
};

template <int D, int HPW>
__global__ __launch_bounds__(kWaves * 64 * HPW) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ out, float* __restrict__ lse, int B, int Hq, int Hkv, int T, int d, float scale_log2,
    int causal, int window) {
  using G = F32Geo<D, HPW>;
  constexpr int kThreads = G::Threads;
  __shared__ __attribute__((aligned(16))) float Ks[kKeys * G::KStride];
  __shared__ __attribute__((aligned(16))) float Vt[D * kVtStride];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;
  const int h = lane >> 5;
  // one-dimensional grid, heaviest q-tiles first across every (batch, head); the
  // workgroups of one (batch, head) keep the residue of their id mod 8, and so their
  // XCD, when B*Hq is a multiple of 8
  const int hgroups = Hq / HPW;  // HPW query heads of one K/V group per workgroup
  const int units = hgroups * B;
  const int qt = (int)(gridDim.x / units) - 1 - (int)blockIdx.x / units;
  const int hq = (int)blockIdx.x % units % hgroups * HPW + wave / kWaves;
  const int b = (int)blockIdx.x % units / hgroups;
  const int g = hq / (Hq / Hkv);
  const int q0 = qt * (kWaves * kRows) + wave % kWaves * kRows;  // the wave's first query row
  const int qi = q0 + col;                              // the lane's query row
  // rows in memory are d floats; D is d rounded up to 32, the padded dims are zeros
  const long long qbase = ((long long)b * Hq + hq) * (long long)T * d;
  const long long kvbase = ((long long)b * Hkv + g) * (long long)T * d;

  // Q^T fragment: head dims h*D/2 .. h*D/2 + D/2 - 1 of the lane's row, times scale*log2(e)
  // so that scores come out in log2 units.  Rows past T are zero (never stored).
  float qf[G::Half];
  {
    const bool ok = qi < T;
    const float* src = q + qbase + (long long)(ok ? qi : 0) * d + h * G::Half;
#pragma unroll
    for (int u = 0; u < G::Half / 4; ++u) {
      f32x4 x = (ok && h * G::Half + 4 * u < d) ? *reinterpret_cast<const f32x4*>(src + 4 * u)
                                                : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * u + e] = x[e] * scale_log2;
    }
  }

  // keys the workgroup walks, and the keys this wave sees (none for a wave past T)
  const int wg_rows_end = min(T, (qt + 1) * kWaves * kRows);
  const int kend = causal ? wg_rows_end : T;
  const int wave_kend = q0 >= T ? 0 : (causal ? min(T, q0 + kRows) : T);
  // with a window: the first tile any row of the workgroup sees, the first key the wave's
  // first row sees, and (below it) the first key every row of the wave sees
  const int kbeg = window > 0 ? max(0, qt * (kWaves * kRows) - window + 1) / kKeys * kKeys : 0;
  const int wave_kbeg = window > 0 ? q0 - window + 1 : 0;
  const int wave_kfull = window > 0 ? q0 + kRows - window : 0;

  // tile staging: chunk c = threadIdx.x + kThreads*i is key c / C4, head dims 4*(c % C4) ..
  f32x4 kr[G::LPT], vr[G::LPT];
  auto load = [&](int j0) {
#pragma unroll
    for (int i = 0; i < G::LPT; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int j = j0 + c / G::C4;
      const int e0 = 4 * (c % G::C4);
      const long long off = kvbase + (long long)j * d + e0;
      if (j < T && e0 < d) {
        kr[i] = *reinterpret_cast<const f32x4*>(k + off);
        vr[i] = *reinterpret_cast<const f32x4*>(v + off);
      } else {
        kr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        vr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < G::LPT; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int key = c / G::C4, e0 = 4 * (c % G::C4);
      *reinterpret_cast<f32x4*>(Ks + key * G::KStride + e0) = kr[i];
#pragma unroll
      for (int u = 0; u < 4; ++u) Vt[(e0 + u) * kVtStride + key] = vr[i][u];
    }
  };

  f32x16 o[G::DB];
#pragma unroll
  for (int db = 0; db < G::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -INFINITY;  // running max of the lane's query (log2 units), shared by both halves
  float l = 0.f;        // this lane's share of the normalizer (its 16 keys of every tile)

  if (kbeg < kend) load(kbeg);
  for (int j0 = kbeg; j0 < kend; j0 += kKeys) {
    __syncthreads();  // every wave is done reading the previous tile
    store();
    __syncthreads();
    if (j0 + kKeys < kend) load(j0 + kKeys);  // in flight during this tile's products
    if (j0 >= wave_kend || j0 + kKeys <= wave_kbeg) continue;  // wave-uniform: no key visible

    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const float* krow = Ks + col * G::KStride + h * G::Half;
#pragma unroll
    for (int u = 0; u < G::Half / 4; ++u) {
      const f32x4 kk = *reinterpret_cast<const f32x4*>(krow + 4 * u);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(kk[e], qf[4 * u + e], s, 0, 0, 0);
    }

    // mask keys past T and, on the diagonal, keys after the query
    if (j0 + kKeys > T || (causal && j0 + kKeys - 1 > q0) || j0 < wave_kfull) {  // wave-uniform
      const int lim = causal ? min(T - 1, qi) : T - 1;  // last key the lane's query sees
      const int lo = window > 0 ? qi - window + 1 : 0;  // first key it sees
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 8 * (r >> 2) + 4 * h + (r & 3);
        s[r] = (key <= lim && key >= lo) ? s[r] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;  // no visible key yet
    const float alpha = __builtin_amdgcn_exp2f(m - m_ref);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(s[r] - m_ref);
      l += p[r];
    }

#pragma unroll
    for (int db = 0; db < G::DB; ++db) {
      const float* vrow = Vt + (32 * db + col) * kVtStride + 4 * h;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const f32x4 vv = *reinterpret_cast<const f32x4*>(vrow + 8 * t4);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[u], p[4 * t4 + u], o[db], 0, 0, 0);
      }
    }
  }

  if (q0 < T) {  // wave-uniform
    const float lt = l + __shfl_xor(l, 32);
    if (qi < T) {
      const float inv = 1.f / lt;
      float* dst = out + qbase + (long long)qi * d;
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          f32x4 x;
#pragma unroll
          for (int u = 0; u < 4; ++u) x[u] = o[db][4 * rr + u] * inv;
          if (32 * db + 8 * rr + 4 * h < d) *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * rr + 4 * h) = x;
        }
      // row log-sum-exp of the scaled scores, natural log
      if (lse && h == 0)
        lse[((long long)b * Hq + hq) * T + qi] = (m + __log2f(lt)) * 0.6931471805599453f;
    }
  }
}

// two query heads per workgroup at d = 128 when the group size is even (see launch_f32)
int f32_hpw(int Hq, int Hkv, int d) { return ((d + 31) / 32 == 4 && (Hq / Hkv) % 2 == 0) ? 2 : 1; }

template <int D, int HPW>
hipError_t launch_f32h(const PrefillArgs& a, hipStream_t stream) {
  const int nqt = (a.T + kWaves * kRows - 1) / (kWaves * kRows);
  dim3 grid(nqt * (a.Hq / HPW) * a.B);  // q-tile-major: every (batch, head group) of the heaviest tile first
  hipLaunchKernelGGL((prefill_f32_kernel<D, HPW>), grid, dim3(kWaves * 64 * HPW), 0, stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), a.out, a.lse, a.B, a.Hq, a.Hkv, a.T, a.d,
                     a.scale * 1.4426950408889634f, a.causal, a.window);
  return hipGetLastError();
}

// d = 128: two query heads of a K/V group share each staged tile when the group size is even
// (+9%; at d = 64 the 512-thread workgroup measured 20% slower and is not used)
template <int D>
hipError_t launch_f32(const PrefillArgs& a, hipStream_t stream) {
  if constexpr (D == 128) {
    if ((a.Hq / a.Hkv) % 2 == 0) return launch_f32h<D, 2>(a, stream);
  }
  return launch_f32h<D, 1>(a, stream);
}

}  // namespace

long long prefill_f32_mfma_waves(int B, int Hq, int Hkv, int T, int d) {
  const int hpw = f32_hpw(Hq, Hkv, d);
  return (long long)((T + kWaves * kRows - 1) / (kWaves * kRows)) * (Hq / hpw) * B * kWaves * hpw;
}

bool prefill_f32_mfma_supported(int d, int Hq, int Hkv) {
  return d > 0 && d <= 128 && d % 16 == 0 && Hkv > 0 && Hq % Hkv == 0;
}

hipError_t launch_attn_prefill_f32_mfma(const PrefillArgs& a, hipStream_t stream) {
  switch ((a.d + 31) / 32) {  // d a multiple of 16, padded to the next multiple of 32
    case 1: return launch_f32<32>(a, stream);
    case 2: return launch_f32<64>(a, stream);
    case 3: return launch_f32<96>(a, stream);
    case 4: return launch_f32<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
