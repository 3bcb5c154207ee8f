// launch.h -- internal interface between the C ABI (api.hip) and the kernels.
// Not installed; the public interface is include/gqa_attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// Generic vector-ALU kernel: q/out rows addressed by strides (elements), so one
// kernel serves the head-major prefill layout and the token-major decode layout.
// k, v are [B, Hkv, Tk, d].  Query row i is at absolute position pos0 + i.
struct GenericArgs {
  const void* q;
  const void* k;
  const void* v;
  float* out;
  int dtype;
  int B, Hq, Hkv, Tq, Tk, d;
  float scale;
  int causal;
  int pos0;
  long long q_sb, q_sh, q_st;  // strides of q and out: batch, head, row
  int window;                  // local window (causal only); 0 = none
  float* lse;                  // [B, Hq, Tq] row log-sum-exp (natural log), or nullptr
};
hipError_t launch_attn_generic(const GenericArgs& a, hipStream_t stream);

// bf16 matrix-core prefill: q/out [B,Hq,T,d], k/v [B,Hkv,T,d], d in {16,...,128} step 16.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  float* out;
  int B, Hq, Hkv, T, d;
  float scale;
  int causal;
  int window;  // local window (causal only); 0 = none
  float* lse;  // [B, Hq, T] row log-sum-exp (natural log), or nullptr
};
bool prefill_mfma_supported(int dtype, int d, int Hq, int Hkv);
hipError_t launch_attn_prefill_mfma(const PrefillArgs& a, hipStream_t stream);
// Workgroups prefill_mfma launches for the shape: fewer than the CU count leaves the
// chip partly idle, and the split-key kernel below serves such shapes.
long long prefill_mfma_grid(int B, int Hq, int Hkv, int T);
// bf16 matrix-core prefill with each 32-row slice's keys split over the waves of its
// workgroup (no local window); same shapes as prefill_mfma.
hipError_t launch_attn_prefill_small(const PrefillArgs& a, hipStream_t stream);
// fp32 matrix-core prefill (the same PrefillArgs, fp32 q/k/v): d a multiple of 16, <= 128.
bool prefill_f32_mfma_supported(int d, int Hq, int Hkv);
hipError_t launch_attn_prefill_f32_mfma(const PrefillArgs& a, hipStream_t stream);
// Waves prefill_f32_mfma launches for the shape.
long long prefill_f32_mfma_waves(int B, int Hq, int Hkv, int T, int d);
// fp32 matrix-core prefill with each 32-row slice's keys split over the waves of its
// workgroup (no local window); same shapes as prefill_f32_mfma.
hipError_t launch_attn_prefill_f32_small(const PrefillArgs& a, hipStream_t stream);

// Split-KV decode plan, a pure function of the shape.
struct DecodePlan {
  int nsplit;        // key chunks per (sequence, kv head); 1 = no split
  int chunk;         // keys per chunk (multiple of the kernel's key tile)
  size_t workspace;  // bytes of partial results
  bool mfma;         // the bf16 matrix-core decode kernel applies
};
// `span` is the most keys one sequence's new tokens can see: the history length, or
// with a local window W at most W + n - 1 (+ alignment, see decode_key_span).
DecodePlan plan_decode(int B, int n, int span, int Hq, int Hkv, int d, int dtype);
// Keys the split kernel walks for a history of `len` positions with n new tokens and
// local window `window` (0 = none): the window's first key rounded down to the
// 32-key tile, up to len.  The host bound for paged decode uses len = max_len.
int decode_key_span(int len, int n, int window);

struct DecodeArgs {
  const void* q;   // [B, n, Hq, d]
  const void* kc;  // [B, Hkv, L, d]
  const void* vc;
  float* out;      // [B, n, Hq, d]
  int B, n, Hq, Hkv, L, d, start_pos;
  float scale;
  void* workspace;
  int window;      // local window; 0 = none
};
hipError_t launch_attn_decode_mfma(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream);
// Device address of the fixed scratch array of attn_decode_cached_noalloc on the current
// device (GQA_NOALLOC_SCRATCH_BYTES); a gqa_status code.
int noalloc_scratch(void** ptr);

// Paged history: kc/vc of DecodeArgs are the block pools, [num_blocks, Hkv, block_size, d]
// (head-major blocks) or [num_blocks, block_size, Hkv, d] (token_major); L and start_pos
// of DecodeArgs are unused (each sequence has its own length).
struct PagedArgs {
  const int* table;     // [B, max_blocks], device
  const int* seq_lens;  // [B], device
  int block_size, max_blocks, num_blocks;
  bool token_major;
};
hipError_t launch_attn_decode_paged(const DecodeArgs& a, const PagedArgs& pg, const DecodePlan& p,
                                    hipStream_t stream);

// KV-cache append with NeoX RoPE on K.  k_new/v_new [B, n, Hkv, d] fp32; kc/vc the cache
// [B, Hkv, L, d] (table == nullptr, rows start_pos..) or the paged pools
// [num_blocks, Hkv, block_size, d] (rows seq_lens[b]-n.. through the block table).
// d is a multiple of 8.  rope = 0 writes K unrotated.
struct KvAppendArgs {
  const float* k_new;
  const float* v_new;
  void* kc;
  void* vc;
  const float* freq_factors;  // [d/2] or nullptr
  int dtype;                  // of the cache
  int B, n, Hkv, d;
  int L, start_pos;                                // contiguous cache
  const int* table;                                // paged: [B, max_blocks], or nullptr
  const int* seq_lens;                             // paged: [B]
  int block_size, max_blocks, num_blocks;          // paged
  int rope;
  double inv_freq[128];                            // base^(-2j/d), j < d/2 (rope only)
};
hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream);

// Backward pass of causal GQA prefill on bf16 matrix cores.  q/out/dout/dq [B,Hq,T,d],
// k/v/dk/dv [B,Hkv,T,d], lse [B,Hq,T] (natural log, from the forward pass); d a
// multiple of 16, <= 128.  dob, lse2, Dv point into the workspace.
struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* out;
  const float* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  int B, Hq, Hkv, T, d;
  float scale;
  int causal;
  uint16_t* dob;  // [B,Hq,T,d] dO rounded to bf16
  float* lse2;    // [B,Hq,T] lse in log2 units
  float* Dv;      // [B,Hq,T] rowsum(dO * O)
};
size_t backward_workspace_bytes(int B, int Hq, int T, int d);
hipError_t launch_attn_backward_mfma(BackwardArgs a, void* workspace, hipStream_t stream);
// Vector-ALU backward: fp32 or bf16 (dtype), any d <= 256; lse2 and Dv in the workspace.
size_t backward_generic_workspace_bytes(int B, int Hq, int T);
hipError_t launch_attn_backward_generic(BackwardArgs a, void* workspace, int dtype, hipStream_t stream);

}  // namespace gqa
