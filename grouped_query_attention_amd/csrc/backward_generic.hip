// backward_generic.hip -- vector-ALU backward pass of causal GQA attention for what the
// matrix-core backward does not cover: fp32 inputs (Riftco's memory-linear path trains
// in float32) and bf16 head dims that are not a multiple of 16, any head dim up to 256.
//
// The same recomputation as the matrix-core path (Riftco, "Two exact full-sequence
// algorithms"): P_ij = exp(s_ij - lse_i) from the saved row statistic, D_i = dO_i . O_i,
// dS_ij = P_ij (dO_i . v_j - D_i), dQ_i = scale sum_j dS_ij k_j, dK_j = scale sum_i dS_ij q_i,
// dV_j = sum_i P_ij dO_i, with the K/V sums running over every query head of the group.
//
// Work split, the forward generic kernel's: a 256-thread block owns 32 rows (query rows
// for dQ, key rows for dK/dV), each row served by 8 lanes holding DPL head dims (dims
// c, c+8, ... for lane c).  The other side's rows are staged through LDS in fp32, 32 at
// a time; dot products reduce over the 8 lanes with three xor-shuffles.  Two kernels, no
// atomics: the result is deterministic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"

namespace gqa {
namespace {

constexpr int kLanes = 8;
constexpr int kRows = 256 / kLanes;  // 32 rows per block
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ float row_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x;
}

// per row: D = dO . O (fp32) and the lse in log2 units
__global__ __launch_bounds__(256) void bwd_gen_prep_kernel(const float* __restrict__ out,
                                                           const float* __restrict__ dout,
                                                           const float* __restrict__ lse,
                                                           float* __restrict__ lse2, float* __restrict__ Dv,
                                                           long long rows, int d) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float acc = 0.f;
  for (int e = lane; e < d; e += 64) acc += dout[row * d + e] * out[row * d + e];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) {
    Dv[row] = acc;
    lse2[row] = lse[row] * kLog2e;
  }
}

template <typename E, int DPL>
__global__ __launch_bounds__(256) void bwd_gen_dq_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                         const E* __restrict__ v, const float* __restrict__ dout,
                                                         const float* __restrict__ lse2,
                                                         const float* __restrict__ Dv, float* __restrict__ dq,
                                                         int B, int Hq, int Hkv, int T, int d, float c, float scale,
                                                         int causal) {
  constexpr int DP = DPL * kLanes;
  __shared__ float Ks[kRows * DP];
  __shared__ float Vs[kRows * DP];
  const int tid = threadIdx.x, r = tid / kLanes, cl = tid % kLanes;
  // one-dimensional grid: the last row block (the most keys) of every (batch, head) first
  const int units = Hq * B;
  const int rb = (int)(gridDim.x / units) - 1 - (int)blockIdx.x / units;
  const int h = (int)blockIdx.x % units % Hq, b = (int)blockIdx.x % units / Hq, g = h / (Hq / Hkv);
  const int i = rb * kRows + r;
  const bool row_ok = i < T;
  const long long row = ((long long)b * Hq + h) * T + i;
  const long long kvoff = ((long long)b * Hkv + g) * (long long)T * d;

  float qr[DPL], gr[DPL], acc[DPL];
#pragma unroll
  for (int u = 0; u < DPL; ++u) {
    const int e = cl + kLanes * u;
    const bool ok = row_ok && e < d;
    qr[u] = ok ? to_f32(q[row * d + e]) : 0.f;
    gr[u] = ok ? dout[row * d + e] : 0.f;
    acc[u] = 0.f;
  }
  const float l2 = row_ok ? lse2[row] : 0.f;
  const float Di = row_ok ? Dv[row] : 0.f;
  // keys the block's rows can see
  const int kv_lim = causal ? min(T, rb * kRows + kRows) : T;

  for (int j0 = 0; j0 < kv_lim; j0 += kRows) {
    __syncthreads();
    for (int idx = tid; idx < kRows * DP; idx += 256) {
      const int jj = idx / DP, e = idx % DP;
      const bool ok = j0 + jj < kv_lim && e < d;
      const long long gi = kvoff + (long long)(j0 + jj) * d + e;
      Ks[idx] = ok ? to_f32(k[gi]) : 0.f;
      Vs[idx] = ok ? to_f32(v[gi]) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int jj = 0; jj < kRows; ++jj) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int u = 0; u < DPL; ++u) {
        s += qr[u] * Ks[jj * DP + cl + kLanes * u];
        dp += gr[u] * Vs[jj * DP + cl + kLanes * u];
      }
      s = row_sum(s);
      dp = row_sum(dp);
      const int j = j0 + jj;
      const bool allowed = row_ok && j < kv_lim && (!causal || j <= i);
      const float p = allowed ? __builtin_amdgcn_exp2f(s * c - l2) : 0.f;
      const float ds = p * (dp - Di);
#pragma unroll
      for (int u = 0; u < DPL; ++u) acc[u] += ds * Ks[jj * DP + cl + kLanes * u];
    }
  }
  if (row_ok) {
#pragma unroll
    for (int u = 0; u < DPL; ++u) {
      const int e = cl + kLanes * u;
      if (e < d) dq[row * d + e] = acc[u] * scale;
    }
  }
}

template <typename E, int DPL>
__global__ __launch_bounds__(256) void bwd_gen_dkdv_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                           const E* __restrict__ v,
                                                           const float* __restrict__ dout,
                                                           const float* __restrict__ lse2,
                                                           const float* __restrict__ Dv, float* __restrict__ dk,
                                                           float* __restrict__ dv, int B, int Hq, int Hkv, int T,
                                                           int d, float c, float scale, int causal) {
  constexpr int DP = DPL * kLanes;
  __shared__ float Qs[kRows * DP];
  __shared__ float Gs[kRows * DP];
  __shared__ float L2s[kRows];
  __shared__ float Ds[kRows];
  const int tid = threadIdx.x, r = tid / kLanes, cl = tid % kLanes;
  // one-dimensional grid: the first key block (the most queries) of every (batch, K/V head) first
  const int units = Hkv * B;
  const int kb = (int)blockIdx.x / units;
  const int g = (int)blockIdx.x % units % Hkv, b = (int)blockIdx.x % units / Hkv;
  const int G = Hq / Hkv;
  const int j = kb * kRows + r;  // this row's key
  const bool key_ok = j < T;
  const long long krow = ((long long)b * Hkv + g) * T + j;

  float kr[DPL], vr[DPL], ak[DPL], av[DPL];
#pragma unroll
  for (int u = 0; u < DPL; ++u) {
    const int e = cl + kLanes * u;
    const bool ok = key_ok && e < d;
    kr[u] = ok ? to_f32(k[krow * d + e]) : 0.f;
    vr[u] = ok ? to_f32(v[krow * d + e]) : 0.f;
    ak[u] = 0.f;
    av[u] = 0.f;
  }
  // query rows before the block's first key see none of its keys
  const int i_beg = causal ? kb * kRows : 0;
  for (int hq = g * G; hq < g * G + G; ++hq) {
    const long long qbase = ((long long)b * Hq + hq) * T;
    for (int i0 = i_beg; i0 < T; i0 += kRows) {
      __syncthreads();
      for (int idx = tid; idx < kRows * DP; idx += 256) {
        const int ii = idx / DP, e = idx % DP;
        const bool ok = i0 + ii < T && e < d;
        const long long gi = (qbase + i0 + ii) * d + e;
        Qs[idx] = ok ? to_f32(q[gi]) : 0.f;
        Gs[idx] = ok ? dout[gi] : 0.f;
      }
      if (tid < kRows) {
        const bool ok = i0 + tid < T;
        L2s[tid] = ok ? lse2[qbase + i0 + tid] : 0.f;
        Ds[tid] = ok ? Dv[qbase + i0 + tid] : 0.f;
      }
      __syncthreads();
#pragma unroll 4
      for (int ii = 0; ii < kRows; ++ii) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int u = 0; u < DPL; ++u) {
          s += kr[u] * Qs[ii * DP + cl + kLanes * u];
          dp += vr[u] * Gs[ii * DP + cl + kLanes * u];
        }
        s = row_sum(s);
        dp = row_sum(dp);
        const int i = i0 + ii;
        const bool allowed = key_ok && i < T && (!causal || j <= i);
        const float p = allowed ? __builtin_amdgcn_exp2f(s * c - L2s[ii]) : 0.f;
        const float ds = p * (dp - Ds[ii]);
#pragma unroll
        for (int u = 0; u < DPL; ++u) {
          av[u] += p * Gs[ii * DP + cl + kLanes * u];
          ak[u] += ds * Qs[ii * DP + cl + kLanes * u];
        }
      }
    }
  }
  if (key_ok) {
#pragma unroll
    for (int u = 0; u < DPL; ++u) {
      const int e = cl + kLanes * u;
      if (e < d) {
        dk[krow * d + e] = ak[u] * scale;
        dv[krow * d + e] = av[u];
      }
    }
  }
}

template <typename E, int DPL>
hipError_t launch_t(const BackwardArgs& a, hipStream_t s) {
  const float c = a.scale * kLog2e;
  const long long nb = (a.T + kRows - 1) / kRows;
  if (nb * a.Hq * a.B > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_gen_dq_kernel<E, DPL>), dim3((unsigned)(nb * a.Hq * a.B)), dim3(256), 0, s,
                     static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.v), a.dout,
                     a.lse2, a.Dv, a.dq, a.B, a.Hq, a.Hkv, a.T, a.d, c, a.scale, a.causal);
  hipLaunchKernelGGL((bwd_gen_dkdv_kernel<E, DPL>), dim3((unsigned)(nb * a.Hkv * a.B)), dim3(256), 0, s,
                     static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.v), a.dout,
                     a.lse2, a.Dv, a.dk, a.dv, a.B, a.Hq, a.Hkv, a.T, a.d, c, a.scale, a.causal);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_dt(const BackwardArgs& a, hipStream_t s) {
  const int dpl = (a.d + kLanes - 1) / kLanes;
  if (dpl <= 1) return launch_t<E, 1>(a, s);
  if (dpl <= 2) return launch_t<E, 2>(a, s);
  if (dpl <= 4) return launch_t<E, 4>(a, s);
  if (dpl <= 8) return launch_t<E, 8>(a, s);
  if (dpl <= 16) return launch_t<E, 16>(a, s);
  return launch_t<E, 32>(a, s);
}

}  // namespace

hipError_t launch_attn_backward_generic(BackwardArgs a, void* workspace, int dtype, hipStream_t stream) {
  const long long rows = (long long)a.B * a.Hq * a.T;
  char* ws = static_cast<char*>(workspace);
  const size_t fb = ((size_t)rows * 4 + 255) / 256 * 256;
  a.lse2 = reinterpret_cast<float*>(ws);
  a.Dv = reinterpret_cast<float*>(ws + fb);
  const long long pb = (rows + 3) / 4;
  if (pb > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_gen_prep_kernel, dim3((unsigned)pb), dim3(256), 0, stream, a.out, a.dout, a.lse,
                     a.lse2, a.Dv, rows, a.d);
  return dtype == kF32 ? launch_dt<float>(a, stream) : launch_dt<uint16_t>(a, stream);
}

size_t backward_generic_workspace_bytes(int B, int Hq, int T) {
  const size_t rows = (size_t)B * Hq * T;
  return 2 * ((rows * 4 + 255) / 256 * 256);
}

}  // namespace gqa
