// api.hip -- the C ABI declared in include/gqa_attn.h: argument validation on the host,
// kernel choice, and launch on the caller's stream.  Nothing here allocates, frees or
// synchronizes.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gqa_attn.h"
#include "launch.h"

namespace {

constexpr int kMaxHeadDim = 256;
constexpr long long kMaxSeq = 1LL << 30;
// every grid is one-dimensional and decodes (batch, head) from a 32-bit block index
constexpr long long kMaxBatchHeads = 0x7fffffffLL;
constexpr int kCUs = 256;  // compute units of the MI355X
// fp32: the split-key kernel when the one-workgroup-per-q-tile kernel would launch fewer
// waves than four per SIMD (its heaviest q-tile's waves then set the time)
constexpr long long kF32SplitBelowWaves = 4 * 4 * kCUs;

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int dtype, int B, int Hq, int Hkv, int d_h) {
  if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_EINVAL;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || d_h <= 0) return GQA_EINVAL;
  if (Hq % Hkv != 0) return GQA_EINVAL;
  if (d_h > kMaxHeadDim) return GQA_EUNSUPPORTED;
  if ((long long)B * Hq > kMaxBatchHeads) return GQA_EUNSUPPORTED;
  return GQA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_EHIP; }

int prefill_impl(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                 int T, int d_h, float scale, int causal, int window, int dtype, int algo,
                 void* stream, float* lse = nullptr) {
  int rc = check_common(dtype, B, Hq, Hkv, d_h);
  if (rc != GQA_OK) return rc;
  if (T < 0 || !isfinite(scale) || (causal != 0 && causal != 1)) return GQA_EINVAL;
  if (window < 0 || (window > 0 && !causal)) return GQA_EINVAL;
  if (algo != GQA_ALGO_AUTO && algo != GQA_ALGO_GENERIC && algo != GQA_ALGO_MFMA &&
      algo != GQA_ALGO_MFMA_SPLIT)
    return GQA_EINVAL;
  if (T > kMaxSeq) return GQA_EUNSUPPORTED;
  // an explicit kernel request is checked even for empty tensors, so a zero-size call
  // tells the caller whether that kernel covers the shape
  const bool mfma_ok = dtype == GQA_F32
                           ? gqa::prefill_f32_mfma_supported(d_h, Hq, Hkv)
                           : gqa::prefill_mfma_supported(dtype, d_h, Hq, Hkv);
  if (algo == GQA_ALGO_MFMA && !mfma_ok) return GQA_EUNSUPPORTED;
  // the split-key kernels: no local window
  const bool split_ok = mfma_ok && (window == 0 || window >= T);
  if (algo == GQA_ALGO_MFMA_SPLIT && !split_ok) return GQA_EUNSUPPORTED;
  if (B == 0 || T == 0) return GQA_OK;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return GQA_EINVAL;

  hipStream_t s = static_cast<hipStream_t>(stream);
  // a window reaching back to key 0 from every row is plain causal attention: take the
  // same kernel, so the two calls agree bit for bit
  if (window >= T) window = 0;
  gqa::PrefillArgs a{q, k, v, out, B, Hq, Hkv, T, d_h, scale, causal, window, lse};
  // automatic choice: the split-key kernel when one workgroup per q-tile would leave
  // the chip short of work (bf16: fewer workgroups than the 256 CUs)
  const bool small_grid = dtype == GQA_F32
                              ? gqa::prefill_f32_mfma_waves(B, Hq, Hkv, T, d_h) < kF32SplitBelowWaves
                              : gqa::prefill_mfma_grid(B, Hq, Hkv, T) < kCUs;
  if (algo == GQA_ALGO_MFMA_SPLIT || (algo == GQA_ALGO_AUTO && split_ok && small_grid))
    return status_of(dtype == GQA_F32 ? gqa::launch_attn_prefill_f32_small(a, s)
                                      : gqa::launch_attn_prefill_small(a, s));
  if (algo == GQA_ALGO_MFMA || (algo == GQA_ALGO_AUTO && mfma_ok)) {
    if (dtype == GQA_F32) return status_of(gqa::launch_attn_prefill_f32_mfma(a, s));
    return status_of(gqa::launch_attn_prefill_mfma(a, s));
  }
  const long long sd = d_h;
  gqa::GenericArgs ga{q, k, v, out, dtype, B, Hq, Hkv, T, T, d_h, scale, causal, 0,
                      (long long)Hq * T * sd, (long long)T * sd, sd, window, lse};
  return status_of(gqa::launch_attn_generic(ga, s));
}

bool aligned4(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Host-side checks of attn_decode_paged (the device-side table and lengths are checked
// by the kernels).
int paged_check(int B, int newTokens, int Hq, int Hkv, int d_h, int block_size, int max_blocks,
                int num_blocks, int dtype) {
  int rc = check_common(dtype, B, Hq, Hkv, d_h);
  if (rc != GQA_OK) return rc;
  if (newTokens < 0) return GQA_EINVAL;
  const bool empty = B == 0 || newTokens == 0;
  if (!empty && (block_size <= 0 || max_blocks <= 0 || num_blocks <= 0)) return GQA_EINVAL;
  if (block_size < 0 || max_blocks < 0 || num_blocks < 0) return GQA_EINVAL;
  if ((long long)max_blocks * block_size > kMaxSeq) return GQA_EINVAL;
  if (dtype != GQA_BF16 || d_h % 16 != 0 || d_h > 128) return GQA_EUNSUPPORTED;
  if (!empty && block_size % 16 != 0) return GQA_EUNSUPPORTED;
  return GQA_OK;
}

int decode_check(int newTokens, int totalLen, int startPos, int Hq, int Hkv, int d_h, int B,
                 int dtype) {
  int rc = check_common(dtype, B, Hq, Hkv, d_h);
  if (rc != GQA_OK) return rc;
  if (newTokens < 0 || totalLen < 0 || startPos < 0) return GQA_EINVAL;
  if ((long long)startPos + newTokens > totalLen) return GQA_EINVAL;
  if (totalLen > kMaxSeq) return GQA_EUNSUPPORTED;
  return GQA_OK;
}

size_t decode_ws_impl(int B, int newTokens, int totalLen, int Hq, int Hkv, int d_h,
                             int window, int dtype) {
  if (decode_check(newTokens, totalLen, totalLen - newTokens, Hq, Hkv, d_h, B, dtype) != GQA_OK)
    return 0;
  if (window < 0 || B == 0 || newTokens == 0) return 0;
  return gqa::plan_decode(B, newTokens, gqa::decode_key_span(totalLen, newTokens, window), Hq, Hkv,
                          d_h, dtype)
      .workspace;
}

int decode_impl(const void* q, const void* kcache, const void* vcache, float* out,
                       int newTokens, int totalLen, int startPos, int Hq, int Hkv, int d_h, int B,
                       int window, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int rc = decode_check(newTokens, totalLen, startPos, Hq, Hkv, d_h, B, dtype);
  if (rc != GQA_OK) return rc;
  if (window < 0) return GQA_EINVAL;
  if (B == 0 || newTokens == 0) return GQA_OK;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(out))
    return GQA_EINVAL;
  const gqa::DecodePlan plan = gqa::plan_decode(
      B, newTokens, gqa::decode_key_span(totalLen, newTokens, window), Hq, Hkv, d_h, dtype);
  if (plan.workspace > 0 && (workspace == nullptr || workspace_bytes < plan.workspace))
    return GQA_EWORKSPACE;
  if (plan.workspace > 0 && !aligned16(workspace)) return GQA_EINVAL;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale = 1.0f / sqrtf((float)d_h);
  if (plan.mfma) {
    gqa::DecodeArgs a{q, kcache, vcache, out, B, newTokens, Hq, Hkv, totalLen, d_h, startPos,
                      scale, workspace, window};
    return status_of(gqa::launch_attn_decode_mfma(a, plan, s));
  }
  const long long sd = d_h;
  gqa::GenericArgs a{q, kcache, vcache, out, dtype, B, Hq, Hkv, newTokens, totalLen, d_h, scale,
                     1, startPos, (long long)newTokens * Hq * sd, sd, (long long)Hq * sd, window, nullptr};
  return status_of(gqa::launch_attn_generic(a, s));
}

size_t paged_ws_impl(int B, int newTokens, int Hq, int Hkv, int d_h, int block_size,
                            int max_blocks, int window, int dtype) {
  if (paged_check(B, newTokens, Hq, Hkv, d_h, block_size, max_blocks, 1, dtype) != GQA_OK)
    return 0;
  if (window < 0 || B == 0 || newTokens == 0) return 0;
  return gqa::plan_decode(B, newTokens,
                          gqa::decode_key_span(block_size * max_blocks, newTokens, window), Hq,
                          Hkv, d_h, dtype)
      .workspace;
}

int paged_impl(const void* q, const void* kpool, const void* vpool,
                      const int* block_table, const int* seq_lens, float* out, int B,
                      int newTokens, int Hq, int Hkv, int d_h, int block_size, int max_blocks,
                      int num_blocks, int window, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream, bool token_major = false) {
  int rc = paged_check(B, newTokens, Hq, Hkv, d_h, block_size, max_blocks, num_blocks, dtype);
  if (rc != GQA_OK) return rc;
  if (window < 0) return GQA_EINVAL;
  if (B == 0 || newTokens == 0) return GQA_OK;
  if (!aligned16(q) || !aligned16(kpool) || !aligned16(vpool) || !aligned16(out) ||
      !aligned4(block_table) || !aligned4(seq_lens))
    return GQA_EINVAL;
  const int max_len = block_size * max_blocks;
  const gqa::DecodePlan plan = gqa::plan_decode(
      B, newTokens, gqa::decode_key_span(max_len, newTokens, window), Hq, Hkv, d_h, dtype);
  if (!plan.mfma) return GQA_EUNSUPPORTED;
  if (plan.workspace > 0 && (workspace == nullptr || workspace_bytes < plan.workspace))
    return GQA_EWORKSPACE;
  if (plan.workspace > 0 && !aligned16(workspace)) return GQA_EINVAL;
  gqa::DecodeArgs a{q, kpool, vpool, out, B, newTokens, Hq, Hkv, max_len, d_h, 0,
                    1.0f / sqrtf((float)d_h), workspace, window};
  gqa::PagedArgs pg{block_table, seq_lens, block_size, max_blocks, num_blocks, token_major};
  return status_of(gqa::launch_attn_decode_paged(a, pg, plan, static_cast<hipStream_t>(stream)));
}

// Inverse frequencies of the rotation pairs, base^(-2j/d) in double (the kernel divides
// by the per-pair factors and multiplies by the position).
void fill_inv_freq(gqa::KvAppendArgs& a, float rope_base) {
  if (!a.rope) return;
  for (int j = 0; j < a.d / 2; ++j) a.inv_freq[j] = pow((double)rope_base, -2.0 * j / a.d);
}

// Host checks shared by both append entry points.
int append_check(const float* k_new, const float* v_new, const void* kc, const void* vc,
                 const float* freq_factors, int B, int newTokens, int Hkv, int d_h, float rope_base,
                 int dtype) {
  if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_EINVAL;
  if (B < 0 || newTokens < 0 || Hkv <= 0 || d_h <= 0) return GQA_EINVAL;
  if (!(rope_base >= 0.f) || !isfinite(rope_base)) return GQA_EINVAL;
  if (d_h > kMaxHeadDim || d_h % 8 != 0) return GQA_EUNSUPPORTED;
  if (B == 0 || newTokens == 0) return GQA_OK;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(kc) || !aligned16(vc)) return GQA_EINVAL;
  if (freq_factors && rope_base > 0.f && !aligned4(freq_factors)) return GQA_EINVAL;
  return GQA_OK;
}

}  // namespace

extern "C" {

int attn_prefill(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                 int T, int d_h, float scale, int causal, int dtype, void* stream) {
  return prefill_impl(q, k, v, out, B, Hq, Hkv, T, d_h, scale, causal, 0, dtype, GQA_ALGO_AUTO,
                      stream);
}

int attn_prefill_ex(const void* q, const void* k, const void* v, float* out, int B, int Hq,
                    int Hkv, int T, int d_h, float scale, int causal, int dtype, int algo,
                    void* stream) {
  return prefill_impl(q, k, v, out, B, Hq, Hkv, T, d_h, scale, causal, 0, dtype, algo, stream);
}

int attn_prefill_lse(const void* q, const void* k, const void* v, float* out, float* lse, int B, int Hq,
                     int Hkv, int T, int d_h, float scale, int causal, int dtype, void* stream) {
  if (B > 0 && T > 0 && !aligned4(lse)) return GQA_EINVAL;
  return prefill_impl(q, k, v, out, B, Hq, Hkv, T, d_h, scale, causal, 0, dtype, GQA_ALGO_AUTO, stream, lse);
}

int attn_prefill_window(const void* q, const void* k, const void* v, float* out, int B, int Hq,
                        int Hkv, int T, int d_h, float scale, int window, int dtype, void* stream) {
  if (window < 1) return GQA_EINVAL;
  return prefill_impl(q, k, v, out, B, Hq, Hkv, T, d_h, scale, 1, window, dtype, GQA_ALGO_AUTO,
                      stream);
}

size_t attn_decode_workspace_bytes(int B, int newTokens, int totalLen, int Hq, int Hkv, int d_h,
                                   int dtype) {
  return decode_ws_impl(B, newTokens, totalLen, Hq, Hkv, d_h, 0, dtype);
}


int attn_decode_num_splits(int B, int newTokens, int totalLen, int Hq, int Hkv, int d_h,
                           int dtype) {
  if (decode_check(newTokens, totalLen, totalLen - newTokens, Hq, Hkv, d_h, B, dtype) != GQA_OK)
    return 0;
  if (B == 0 || newTokens == 0) return 0;
  return gqa::plan_decode(B, newTokens, totalLen, Hq, Hkv, d_h, dtype).nsplit;
}


int attn_decode_cached(const void* q, const void* kcache, const void* vcache, float* out,
                       int newTokens, int totalLen, int startPos, int Hq, int Hkv, int d_h, int B,
                       int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, kcache, vcache, out, newTokens, totalLen, startPos, Hq, Hkv, d_h, B, 0,
                     dtype, workspace, workspace_bytes, stream);
}

size_t attn_decode_window_workspace_bytes(int B, int newTokens, int totalLen, int Hq, int Hkv,
                                          int d_h, int window, int dtype) {
  if (window < 1) return 0;
  return decode_ws_impl(B, newTokens, totalLen, Hq, Hkv, d_h, window, dtype);
}

int attn_decode_window(const void* q, const void* kcache, const void* vcache, float* out,
                       int newTokens, int totalLen, int startPos, int Hq, int Hkv, int d_h, int B,
                       int window, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (window < 1) return GQA_EINVAL;
  return decode_impl(q, kcache, vcache, out, newTokens, totalLen, startPos, Hq, Hkv, d_h, B, window,
                     dtype, workspace, workspace_bytes, stream);
}


int attn_decode_cached_noalloc(const void* q, const void* kcache, const void* vcache, float* out,
                               int newTokens, int totalLen, int startPos, int Hq, int Hkv, int d_h,
                               int B, int dtype, void* stream) {
  // every argument check of attn_decode_cached first: nothing touches the device for a
  // call that will be rejected
  int rc = decode_check(newTokens, totalLen, startPos, Hq, Hkv, d_h, B, dtype);
  if (rc != GQA_OK) return rc;
  if (B == 0 || newTokens == 0) return GQA_OK;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(out))
    return GQA_EINVAL;
  const size_t need = gqa::plan_decode(B, newTokens, totalLen, Hq, Hkv, d_h, dtype).workspace;
  if (need > GQA_NOALLOC_SCRATCH_BYTES) return GQA_ESCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    rc = gqa::noalloc_scratch(&ws);
    if (rc != GQA_OK) return rc;
  }
  return decode_impl(q, kcache, vcache, out, newTokens, totalLen, startPos, Hq, Hkv, d_h, B, 0,
                     dtype, ws, need > 0 ? GQA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

size_t attn_decode_paged_workspace_bytes(int B, int newTokens, int Hq, int Hkv, int d_h,
                                         int block_size, int max_blocks, int dtype) {
  return paged_ws_impl(B, newTokens, Hq, Hkv, d_h, block_size, max_blocks, 0, dtype);
}

size_t attn_decode_paged_window_workspace_bytes(int B, int newTokens, int Hq, int Hkv, int d_h,
                                                int block_size, int max_blocks, int window,
                                                int dtype) {
  if (window < 1) return 0;
  return paged_ws_impl(B, newTokens, Hq, Hkv, d_h, block_size, max_blocks, window, dtype);
}


int attn_decode_paged(const void* q, const void* kpool, const void* vpool, const int* block_table,
                      const int* seq_lens, float* out, int B, int newTokens, int Hq, int Hkv,
                      int d_h, int block_size, int max_blocks, int num_blocks, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return paged_impl(q, kpool, vpool, block_table, seq_lens, out, B, newTokens, Hq, Hkv, d_h,
                    block_size, max_blocks, num_blocks, 0, dtype, workspace, workspace_bytes,
                    stream);
}

int attn_decode_blocks(const void* q, const void* kpool, const void* vpool, const int* block_table,
                       const int* seq_lens, float* out, int B, int newTokens, int Hq, int Hkv,
                       int d_h, int block_size, int max_blocks, int num_blocks, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return paged_impl(q, kpool, vpool, block_table, seq_lens, out, B, newTokens, Hq, Hkv, d_h,
                    block_size, max_blocks, num_blocks, 0, dtype, workspace, workspace_bytes,
                    stream, true);
}

int attn_decode_paged_window(const void* q, const void* kpool, const void* vpool,
                             const int* block_table, const int* seq_lens, float* out, int B,
                             int newTokens, int Hq, int Hkv, int d_h, int block_size,
                             int max_blocks, int num_blocks, int window, int dtype,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (window < 1) return GQA_EINVAL;
  return paged_impl(q, kpool, vpool, block_table, seq_lens, out, B, newTokens, Hq, Hkv, d_h,
                    block_size, max_blocks, num_blocks, window, dtype, workspace, workspace_bytes,
                    stream);
}

size_t attn_backward_workspace_bytes(int B, int Hq, int Hkv, int T, int d_h, int dtype) {
  if (check_common(dtype, B, Hq, Hkv, d_h) != GQA_OK || T < 0) return 0;
  if (gqa::prefill_mfma_supported(dtype, d_h, Hq, Hkv)) return gqa::backward_workspace_bytes(B, Hq, T, d_h);
  return gqa::backward_generic_workspace_bytes(B, Hq, T);
}

int attn_backward(const void* q, const void* k, const void* v, const float* out, const float* dout,
                  const float* lse, float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int T, int d_h,
                  float scale, int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common(dtype, B, Hq, Hkv, d_h);
  if (rc != GQA_OK) return rc;
  if (T < 0 || !isfinite(scale) || (causal != 0 && causal != 1)) return GQA_EINVAL;
  if (T > kMaxSeq) return GQA_EUNSUPPORTED;
  if (B == 0 || T == 0) return GQA_OK;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned4(lse))
    return GQA_EINVAL;
  const bool mfma = gqa::prefill_mfma_supported(dtype, d_h, Hq, Hkv);
  const size_t need = mfma ? gqa::backward_workspace_bytes(B, Hq, T, d_h)
                           : gqa::backward_generic_workspace_bytes(B, Hq, T);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return GQA_EWORKSPACE;
  gqa::BackwardArgs a{q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, T, d_h, scale, causal,
                      nullptr, nullptr, nullptr};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return status_of(mfma ? gqa::launch_attn_backward_mfma(a, workspace, s)
                        : gqa::launch_attn_backward_generic(a, workspace, dtype, s));
}

int attn_kv_append(const float* k_new, const float* v_new, void* kcache, void* vcache,
                   const float* freq_factors, int B, int newTokens, int Hkv, int d_h, int totalLen,
                   int start_pos, float rope_base, int dtype, void* stream) {
  int rc = append_check(k_new, v_new, kcache, vcache, freq_factors, B, newTokens, Hkv, d_h, rope_base,
                        dtype);
  if (rc != GQA_OK) return rc;
  if (totalLen < 0 || start_pos < 0 || (long long)start_pos + newTokens > totalLen) return GQA_EINVAL;
  if (totalLen > kMaxSeq) return GQA_EUNSUPPORTED;
  if (B == 0 || newTokens == 0) return GQA_OK;
  gqa::KvAppendArgs a{k_new, v_new, kcache, vcache, freq_factors, dtype, B, newTokens, Hkv, d_h,
                      totalLen, start_pos, nullptr, nullptr, 0, 0, 0, rope_base > 0.f ? 1 : 0, {}};
  fill_inv_freq(a, rope_base);
  return status_of(gqa::launch_kv_append(a, static_cast<hipStream_t>(stream)));
}

int attn_kv_append_paged(const float* k_new, const float* v_new, void* kpool, void* vpool,
                         const int* block_table, const int* seq_lens, const float* freq_factors, int B,
                         int newTokens, int Hkv, int d_h, int block_size, int max_blocks,
                         int num_blocks, float rope_base, int dtype, void* stream) {
  int rc = append_check(k_new, v_new, kpool, vpool, freq_factors, B, newTokens, Hkv, d_h, rope_base,
                        dtype);
  if (rc != GQA_OK) return rc;
  if (block_size < 0 || max_blocks < 0 || num_blocks < 0) return GQA_EINVAL;
  if ((long long)max_blocks * block_size > kMaxSeq) return GQA_EINVAL;
  if (B == 0 || newTokens == 0) return GQA_OK;
  if (block_size == 0 || max_blocks == 0 || num_blocks == 0) return GQA_EINVAL;
  if (!aligned4(block_table) || !aligned4(seq_lens)) return GQA_EINVAL;
  gqa::KvAppendArgs a{k_new, v_new, kpool, vpool, freq_factors, dtype, B, newTokens, Hkv, d_h, 0, 0,
                      block_table, seq_lens, block_size, max_blocks, num_blocks, rope_base > 0.f ? 1 : 0, {}};
  fill_inv_freq(a, rope_base);
  return status_of(gqa::launch_kv_append(a, static_cast<hipStream_t>(stream)));
}

const char* attn_strerror(int code) {
  switch (code) {
    case GQA_OK: return "success";
    case GQA_EINVAL: return "invalid argument";
    case GQA_EUNSUPPORTED: return "unsupported shape or dtype for the built kernels";
    case GQA_EWORKSPACE: return "decode workspace missing or too small";
    case GQA_EHIP: return "HIP runtime error at launch";
    case GQA_ESCRATCH: return "shape needs more than the fixed scratch of attn_decode_cached_noalloc";
    default: return "unknown status code";
  }
}

}  // extern "C"
