// attn_generic.hip -- vector-ALU causal GQA attention for any head dim up to 256.
//
// Covers what the matrix-core kernels do not: fp32 inputs, bf16 with a head dim
// that is not a multiple of 16, and odd shapes.  One kernel serves both modes:
// query row i sits at absolute position pos0 + i (0 for prefill, startPos for
// cached decode) and sees keys j <= pos0 + i when causal, the key limit of
// makarna's CausalAttentionCached; with a local window W it also needs
// j >= pos0 + i - W + 1 (the multi-query primer's local attention, section 4.1).
//
// Work split: a 256-thread block owns 32 query rows of one query head; each row
// is served by 8 lanes, each lane holding DPL consecutive head dims (c*DPL ..
// c*DPL + DPL - 1 for lane c), so its K and V reads from LDS are 16-byte vectors.
// Key/value tiles of 32 keys are staged through LDS in float32 and shared by the
// 32 rows.  Softmax is the online recurrence (running max m and normalizer l in
// log2 units, numerator rescaled when m grows), which equals the materialized
// softmax of Riftco's "Two exact full-sequence algorithms" up to rounding.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace gqa {
namespace {

constexpr int kLanesPerRow = 8;
constexpr int kRowsPerBlock = 256 / kLanesPerRow;  // 32
constexpr int kKeysPerTile = 32;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

template <typename T, int DPL>
__global__ __launch_bounds__(256) void attn_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    float* __restrict__ out, int B, int Hq, int Hkv, int Tq, int Tk, int d, float scale_log2, int causal,
    int pos0, int window, long long q_sb, long long q_sh, long long q_st, float* __restrict__ lse) {
  constexpr int DP = DPL * kLanesPerRow;  // padded head dim held by one row
  __shared__ __attribute__((aligned(16))) float Ks[kKeysPerTile * DP];
  __shared__ __attribute__((aligned(16))) float Vs[kKeysPerTile * DP];

  const int tid = threadIdx.x;
  const int r = tid / kLanesPerRow;  // row within the block
  const int c = tid % kLanesPerRow;  // lane within the row
  // one-dimensional grid: the last row block (the most keys) of every (batch, head) first
  const int units = Hq * B;
  const int rb = (int)(gridDim.x / units) - 1 - (int)blockIdx.x / units;
  const int h = (int)blockIdx.x % units % Hq;
  const int b = (int)blockIdx.x % units / Hq;
  const int g = h / (Hq / Hkv);
  const int row0 = rb * kRowsPerBlock;
  const int i = row0 + r;
  const bool row_ok = i < Tq;
  const long long pos = (long long)pos0 + i;  // absolute position of this row

  const long long qoff = (long long)b * q_sb + (long long)h * q_sh + (long long)i * q_st;
  const long long kvoff = ((long long)b * Hkv + g) * (long long)Tk * d;

  // q pre-multiplied by scale*log2(e): scores come out in log2 units for exp2.
  float qr[DPL], o[DPL];
#pragma unroll
  for (int u = 0; u < DPL; ++u) {
    const int e = c * DPL + u;
    qr[u] = (row_ok && e < d) ? to_f32(q[qoff + e]) * scale_log2 : 0.f;
    o[u] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  // Keys this block can need: all of them, or up to the last row's position, and with
  // a window from the first row's window start.
  const int last_row = min(Tq, row0 + kRowsPerBlock) - 1;
  const long long lim_ll = causal ? min((long long)Tk, (long long)pos0 + last_row + 1) : (long long)Tk;
  const int kv_lim = (int)lim_ll;
  const int kv_beg = window > 0 ? (int)max(0LL, (long long)pos0 + row0 - window + 1) : 0;
  const long long lo = pos - window + 1;  // this row's first visible key (window > 0)

  for (int j0 = kv_beg; j0 < kv_lim; j0 += kKeysPerTile) {
    __syncthreads();
    for (int idx = tid; idx < kKeysPerTile * DP; idx += 256) {
      const int jj = idx / DP, e = idx % DP;
      const bool ok = (j0 + jj < kv_lim) && e < d;
      const long long gi = kvoff + (long long)(j0 + jj) * d + e;
      Ks[idx] = ok ? to_f32(k[gi]) : 0.f;
      Vs[idx] = ok ? to_f32(v[gi]) : 0.f;
    }
    __syncthreads();

    float s[kKeysPerTile];
    float tmax = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kKeysPerTile; ++jj) {
      float part = 0.f;
#pragma unroll
      for (int u = 0; u < DPL; ++u) part += qr[u] * Ks[jj * DP + c * DPL + u];
      // sum over the 8 lanes of the row; every lane ends with the same value
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      part += __shfl_xor(part, 4);
      const int j = j0 + jj;
      const bool allowed = j < kv_lim && (!causal || (long long)j <= pos) && (window <= 0 || j >= lo);
      s[jj] = allowed ? part : -INFINITY;
      tmax = fmaxf(tmax, s[jj]);
    }
    const float m_new = fmaxf(m, tmax);
    // a row with no visible key yet keeps m = -inf; use 0 as the reference then
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_ref);
    l *= alpha;
#pragma unroll
    for (int u = 0; u < DPL; ++u) o[u] *= alpha;
#pragma unroll
    for (int jj = 0; jj < kKeysPerTile; ++jj) {
      const float p = __builtin_amdgcn_exp2f(s[jj] - m_ref);
      l += p;
#pragma unroll
      for (int u = 0; u < DPL; ++u) o[u] += p * Vs[jj * DP + c * DPL + u];
    }
    m = m_new;
  }

  if (row_ok) {
    const float inv = 1.f / l;
    // row log-sum-exp of the scaled scores, natural log: (m + log2 l) * ln 2
    if (lse && c == 0) lse[((long long)b * Hq + h) * Tq + i] = (m + __log2f(l)) * 0.6931471805599453f;
#pragma unroll
    for (int u = 0; u < DPL; ++u) {
      const int e = c * DPL + u;
      if (e < d) out[qoff + e] = o[u] * inv;
    }
  }
}

template <typename T, int DPL>
hipError_t launch_t(const GenericArgs& a, hipStream_t stream) {
  const long long blocks = (long long)((a.Tq + kRowsPerBlock - 1) / kRowsPerBlock) * a.Hq * a.B;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_generic_kernel<T, DPL>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), a.out, a.B, a.Hq, a.Hkv, a.Tq, a.Tk, a.d,
                     a.scale * 1.4426950408889634f, a.causal, a.pos0, a.window, a.q_sb, a.q_sh,
                     a.q_st, a.lse);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dt(const GenericArgs& a, hipStream_t stream) {
  const int dpl = (a.d + kLanesPerRow - 1) / kLanesPerRow;
  if (dpl <= 1) return launch_t<T, 1>(a, stream);
  if (dpl <= 2) return launch_t<T, 2>(a, stream);
  if (dpl <= 4) return launch_t<T, 4>(a, stream);
  if (dpl <= 8) return launch_t<T, 8>(a, stream);
  if (dpl <= 16) return launch_t<T, 16>(a, stream);
  return launch_t<T, 32>(a, stream);
}

}  // namespace

hipError_t launch_attn_generic(const GenericArgs& a, hipStream_t stream) {
  if (a.dtype == kF32) return launch_dt<float>(a, stream);
  return launch_dt<uint16_t>(a, stream);
}

}  // namespace gqa
