// kv_append.hip -- the step right before cached decode: write the new tokens' K and V
// rows into the cache, rotating K with NeoX rotary embedding on the way (Hesper's fused
// RoPE-K + KV-cache-write kernels; forge's apply_rope at offset start_pos followed by
// the cache append).
//
// New token i of sequence b sits at absolute position p (start_pos + i for a contiguous
// cache; seq_lens[b] - newTokens + i for a paged one).  Head dims j and j + d/2 form
// rotation pair j, turned by p * base^(-2j/d) / freq_factors[j].
//
// Mapping: the work is HBM-bound (read two fp32 rows, write two cache rows), so the
// layout decides everything.  A thread owns 4 consecutive pairs (8 head dims: j..j+3 and
// j+d/2..j+d/2+3) of one token and kHeadsPerThread of its K/V heads, so its angles and
// their sines and cosines serve several heads while enough threads stay in flight to
// cover HBM latency.  Sixteen-byte loads of the fp32 rows and 8-byte (bf16) or 16-byte
// (fp32) stores keep every access coalesced: the threads of one token cover a head's row
// contiguously.
//
// Angles are formed in double precision (the position times the pair's inverse
// frequency, computed on the host in double, reduced modulo 2*pi), so their error does
// not grow with the position; the reduced angle's sine and cosine and the rotation
// itself are fp32.  A thread issues its row loads before the angle arithmetic, so the
// two overlap.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"

namespace gqa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kHeadsPerThread = 2;
constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

// cos and sin of the angle of pair j at position p
__device__ __forceinline__ void pair_sincos(long long p, int j, const double* inv_freq,
                                            const float* __restrict__ ff, float& cs, float& sn) {
  double inv = inv_freq[j];
  if (ff) inv /= (double)ff[j];
  const double ang = (double)p * inv;
  // subtract the nearest whole number of turns; the rounded 1/(2 pi) can misplace the
  // quotient only within ~1e-11 of a half turn, where rint's other choice leaves
  // |r| <= pi + 1e-10 -- still an exact argument for sincosf
  const double r = ang - rint(ang * kInvTwoPi) * kTwoPi;
  sincosf((float)r, &sn, &cs);
}

template <bool BF16>
__device__ __forceinline__ void store4(void* base, long long off, f32x4 x) {
  if (BF16) {
    bf16x4 b = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};  // round to nearest even
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(base) + off) = b;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + off) = x;
  }
}

// One thread: token (b, i), pairs 4*t .. 4*t+3, heads kHeadsPerThread*hg ...  PAGED resolves the
// cache row through the block table; a sequence whose length or table entry does not
// fit is not written.
template <bool BF16, bool PAGED>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(KvAppendArgs a) {
  const int half = a.d / 2;
  const int tpt = half / 4;  // threads per (token, head group)
  const int nhg = (a.Hkv + kHeadsPerThread - 1) / kHeadsPerThread;
  const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long unit = gid / tpt;  // (token, head group)
  if (unit >= (long long)a.B * a.n * nhg) return;
  const int t = (int)(gid - unit * tpt);
  const long long tok = unit / nhg;
  const int h0 = (int)(unit - tok * nhg) * kHeadsPerThread;
  const int h1 = min(a.Hkv, h0 + kHeadsPerThread);
  const int b = (int)(tok / a.n), i = (int)(tok - (long long)b * a.n);
  const int j0 = 4 * t;

  long long p;       // absolute position of the token
  long long row0;    // element offset of (head 0, position p, dim 0) in the cache / pool
  long long hstride; // elements between two heads' rows of this position
  if (PAGED) {
    const int len = a.seq_lens[b];
    if (len < a.n || len > (long long)a.max_blocks * a.block_size) return;
    p = (long long)len - a.n + i;
    const int blk = a.table[(long long)b * a.max_blocks + p / a.block_size];
    if (blk < 0 || blk >= a.num_blocks) return;
    hstride = (long long)a.block_size * a.d;
    row0 = ((long long)blk * a.Hkv * a.block_size + p % a.block_size) * a.d;
  } else {
    p = (long long)a.start_pos + i;
    hstride = (long long)a.L * a.d;
    row0 = ((long long)b * a.Hkv * a.L + p) * a.d;
  }

  // the rows' loads go out first, so their latency overlaps the angle arithmetic
  const long long src0 = tok * a.Hkv * a.d;  // [B, n, Hkv, d]: token tok, head 0
  f32x4 k1s[kHeadsPerThread], k2s[kHeadsPerThread], v1s[kHeadsPerThread], v2s[kHeadsPerThread];
#pragma unroll
  for (int hh = 0; hh < kHeadsPerThread; ++hh) {
    const int h = min(h0 + hh, h1 - 1);  // a missing last head re-reads one in bounds
    const long long src = src0 + (long long)h * a.d;
    k1s[hh] = *reinterpret_cast<const f32x4*>(a.k_new + src + j0);
    k2s[hh] = *reinterpret_cast<const f32x4*>(a.k_new + src + half + j0);
    v1s[hh] = *reinterpret_cast<const f32x4*>(a.v_new + src + j0);
    v2s[hh] = *reinterpret_cast<const f32x4*>(a.v_new + src + half + j0);
  }

  float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.rope) {
#pragma unroll
    for (int e = 0; e < 4; ++e) pair_sincos(p, j0 + e, a.inv_freq, a.freq_factors, cs[e], sn[e]);
  }

#pragma unroll
  for (int hh = 0; hh < kHeadsPerThread; ++hh) {
    const int h = h0 + hh;
    if (h >= h1) break;
    const f32x4 k1 = k1s[hh], k2 = k2s[hh], v1 = v1s[hh], v2 = v2s[hh];
    f32x4 r1, r2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r1[e] = k1[e] * cs[e] - k2[e] * sn[e];
      r2[e] = k2[e] * cs[e] + k1[e] * sn[e];
    }
    const long long dst = row0 + (long long)h * hstride;
    store4<BF16>(a.kc, dst + j0, r1);
    store4<BF16>(a.kc, dst + half + j0, r2);
    store4<BF16>(a.vc, dst + j0, v1);
    store4<BF16>(a.vc, dst + half + j0, v2);
  }
}

template <bool PAGED>
hipError_t launch(const KvAppendArgs& a, hipStream_t s) {
  const long long threads = (long long)a.B * a.n * ((a.Hkv + kHeadsPerThread - 1) / kHeadsPerThread) * (a.d / 8);
  const long long blocks = (threads + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.dtype == kBF16)
    hipLaunchKernelGGL((kv_append_kernel<true, PAGED>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((kv_append_kernel<false, PAGED>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream) {
  return a.table ? launch<true>(a, stream) : launch<false>(a, stream);
}

}  // namespace gqa
