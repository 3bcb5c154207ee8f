/*
 * gqa_attn.h -- C ABI of the gfx950 (MI355X) causal grouped-query attention library
 * (libgqa_attn.so).
 *
 * What every entry point computes, per batch b, query head h and query row i:
 *
 *   g     = h / (Hq / Hkv)        query heads are grouped over K/V heads the way
 *                                 repeat_interleave(group_size) lays them out
 *                                 ("Grouped-Query Attention", section 5.1)
 *   p_i   = absolute position of query row i (i in prefill, startPos + i in decode)
 *   s_ij  = scale * <q[b,h,i,:], k[b,g,j,:]>           (Riftco "Causal Multi-Head
 *                                                      Self-Attention", "Dataflow and shapes")
 *   P_ij  = softmax over j of s_ij, with every key j > p_i given probability exactly 0
 *           when causal (Hesper "Attention" page, "Causal Masking")
 *   out[b,h,i,:] = sum_j P_ij * v[b,g,j,:]
 *
 * Conventions shared by all entry points:
 *   - Tensor pointers are DEVICE pointers on the current HIP device, owned by the
 *     caller, contiguous row-major, and 16-byte aligned.  The library never allocates,
 *     frees or synchronizes; inputs are read-only.
 *   - dtype (enum gqa_dtype) is the element type of q, k, v (or q, kcache, vcache);
 *     out is always float32.  Accumulation is float32 in both dtypes.
 *   - stream is a hipStream_t passed as void*; NULL means the default stream.  Work is
 *     enqueued on it and the call returns before it completes.
 *   - Arguments are validated on the host before anything is enqueued.  A bad argument
 *     returns a negative status and enqueues nothing.  Sizes of zero (B, T, newTokens)
 *     return GQA_OK and enqueue nothing.  GQA_EHIP reports a launch error; a fault
 *     inside a kernel surfaces at the caller's next synchronization.
 *   - Calls are re-entrant; concurrent decode calls need distinct workspaces.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gqa_dtype { GQA_F32 = 0, GQA_BF16 = 1 };

enum gqa_status {
    GQA_OK = 0,
    GQA_EINVAL = -1,       /* argument outside the documented domain */
    GQA_EUNSUPPORTED = -2, /* valid, but no kernel is built for it (e.g. d_h > 256) */
    GQA_EWORKSPACE = -3,   /* decode workspace missing or too small */
    GQA_EHIP = -4,         /* the HIP runtime reported an error at launch */
    GQA_ESCRATCH = -5      /* the shape needs more than the fixed scratch of
                              attn_decode_cached_noalloc (GQA_NOALLOC_SCRATCH_BYTES) */
};

/* Size of the fixed device scratch array attn_decode_cached_noalloc keeps its split-KV
 * partials in (one copy per GPU the library runs on, held until the process ends). */
#define GQA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Kernel selection for attn_prefill_ex (attn_prefill always uses GQA_ALGO_AUTO). */
enum gqa_algo {
    GQA_ALGO_AUTO = 0,    /* fastest kernel built for the shape */
    GQA_ALGO_GENERIC = 1, /* vector-ALU kernel: any d_h in [1, 256], fp32 or bf16 */
    GQA_ALGO_MFMA = 2,    /* matrix-core kernel: bf16 with d_h a multiple of 16, <= 128, or
                             fp32 with d_h a multiple of 16, <= 128 (products in fp32) */
    GQA_ALGO_MFMA_SPLIT = 3 /* matrix-core kernel (bf16, or fp32 with fp32 products) that
                               splits each 32-row query slice's keys over the waves of a
                               workgroup and merges their partial softmax states exactly;
                               same head dims as GQA_ALGO_MFMA, no local window.
                               GQA_ALGO_AUTO takes it when one workgroup per q-tile would
                               leave the GPU's CUs short of work (bf16: fewer workgroups
                               than CUs; fp32: fewer than four waves per SIMD). */
};

/*
 * Full-sequence prefill (Riftco "Dataflow and shapes": attention over [B, H, T, d_h];
 * Hesper "Causal Masking" for the mask).
 *
 *   q, out : [B, Hq,  T, d_h]   (q of dtype; out float32)
 *   k, v   : [B, Hkv, T, d_h]   (dtype)
 *   scale  : multiplies q.k (1/sqrt(d_h) in the pages; any finite value accepted)
 *   causal : 1 = key j visible to row i only when j <= i; 0 = every key visible
 *
 * Errors: GQA_EINVAL for B, T < 0; Hq, Hkv <= 0; Hq % Hkv != 0; d_h <= 0; non-finite
 * scale; causal not 0/1; dtype unknown; a NULL or non-16-byte-aligned pointer when the
 * tensor is non-empty.  GQA_EUNSUPPORTED for d_h > 256.
 */
int attn_prefill(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                 int T, int d_h, float scale, int causal, int dtype, void* stream);

/* attn_prefill with an explicit kernel choice (enum gqa_algo).  GQA_ALGO_MFMA on a shape
 * or dtype it does not cover returns GQA_EUNSUPPORTED, also when B or T is 0 (so an
 * empty call with NULL pointers asks whether the kernel covers a shape). */
int attn_prefill_ex(const void* q, const void* k, const void* v, float* out, int B, int Hq,
                    int Hkv, int T, int d_h, float scale, int causal, int dtype, int algo,
                    void* stream);

/*
 * Local (sliding-window) causal prefill: as attn_prefill with causal = 1, except that
 * query row i sees only keys max(0, i - window + 1) .. i (the multi-query primer's
 * local attention, section 4.1: the current position and the previous window-1).
 * window >= T gives plain causal attention.  Keys below every row's window are never
 * read.  Errors as attn_prefill, plus GQA_EINVAL for window < 1.
 */
int attn_prefill_window(const void* q, const void* k, const void* v, float* out, int B, int Hq,
                        int Hkv, int T, int d_h, float scale, int window, int dtype, void* stream);

/*
 * Bytes of device workspace attn_decode_cached needs for this shape (0 when it needs
 * none).  Pure host arithmetic; the same arguments always give the same answer.
 * Returns 0 for arguments attn_decode_cached would reject.  dtype is an argument
 * because the plan depends on it: a bf16 cache runs the split-KV matrix-core kernels,
 * whose chunk partials live in the workspace; an fp32 cache runs the vector kernel,
 * which needs none.
 */
size_t attn_decode_workspace_bytes(int B, int newTokens, int totalLen, int Hq, int Hkv, int d_h,
                                   int dtype);

/* Number of key chunks the decode kernels split each sequence's history into for this
 * shape (1 = no split).  Pure host arithmetic, for diagnostics and tests. */
int attn_decode_num_splits(int B, int newTokens, int totalLen, int Hq, int Hkv, int d_h,
                           int dtype);

/*
 * Cached decode (makarna's CausalAttentionCached; the cache read of the multi-query
 * primer's section 2.4 "Incremental: one token at a time").
 *
 *   q, out          : [B, newTokens, Hq, d_h]  new-token queries, token-major (q of dtype,
 *                     out float32)
 *   kcache, vcache  : [B, Hkv, totalLen, d_h]  full history per sequence, head-major (the
 *                     Hesper KV cache layout), with the new tokens' K/V already written at
 *                     positions startPos .. startPos+newTokens-1
 *   startPos        : absolute position of the first new token; new token i attends to
 *                     keys 0 .. startPos+i (cache rows at or past startPos+newTokens are
 *                     never read, so a larger preallocated cache may hold anything there)
 *   scale           : fixed at 1/sqrt(d_h), as in CausalAttentionCached
 *   workspace       : device buffer of at least attn_decode_workspace_bytes(...) bytes
 *                     (may be NULL when that is 0); contents on entry are ignored
 *
 * Errors: GQA_EINVAL for B, newTokens, totalLen, startPos < 0; startPos+newTokens >
 * totalLen; Hq, Hkv <= 0; Hq % Hkv != 0; d_h <= 0; dtype unknown; NULL or misaligned
 * pointers for non-empty tensors.  GQA_EUNSUPPORTED for d_h > 256.  GQA_EWORKSPACE when
 * workspace_bytes is below the required size or workspace is NULL while it is needed.
 */
int attn_decode_cached(const void* q, const void* kcache, const void* vcache, float* out,
                       int newTokens, int totalLen, int startPos, int Hq, int Hkv, int d_h, int B,
                       int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_cached for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It computes
 * exactly what attn_decode_cached does (same kernels, same split plan, bitwise the same
 * result), but keeps the split-KV partials in a fixed device array of
 * GQA_NOALLOC_SCRATCH_BYTES inside the library instead of a caller workspace.  The
 * caller still passes q, the caches and out.  It never calls hipMalloc, hipFree or any
 * allocating routine; the first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress) and keeps its address.
 *
 * Every call on one GPU shares that GPU's array, so calls that overlap on one GPU
 * (different streams, or different threads, without ordering between them) race and
 * may corrupt each other's results; serialize them.  Nothing in the array needs to
 * start at zero: every partial a call reads was written earlier in the same call.
 * The array keeps the last call's partials.
 *
 * Arguments as attn_decode_cached without the workspace.  Errors as
 * attn_decode_cached, plus GQA_ESCRATCH, returned before anything is enqueued, when
 * attn_decode_workspace_bytes(...) for the shape exceeds GQA_NOALLOC_SCRATCH_BYTES
 * (e.g. 64 or more new tokens for 64 sequences of 32 query heads over a 32768-position
 * history at d_h = 128; up to 63 fit), and GQA_EHIP when the current device or the
 * array's address cannot be obtained.
 */
int attn_decode_cached_noalloc(const void* q, const void* kcache, const void* vcache, float* out,
                               int newTokens, int totalLen, int startPos, int Hq, int Hkv, int d_h,
                               int B, int dtype, void* stream);

/*
 * Local-window cached decode: attn_decode_cached where new token i (position
 * startPos + i) sees only keys startPos + i - window + 1 .. startPos + i.  Only the cache
 * rows from the first new token's window start (rounded down to a multiple of 32) up
 * to startPos + newTokens - 1 are read, and the key split is planned for that span, so
 * the cost follows the window, not the history.  Arguments and errors as
 * attn_decode_cached, plus GQA_EINVAL for window < 1; the workspace is
 * attn_decode_window_workspace_bytes(...) (0 for window < 1 or rejected shapes).
 */
size_t attn_decode_window_workspace_bytes(int B, int newTokens, int totalLen, int Hq, int Hkv,
                                          int d_h, int window, int dtype);
int attn_decode_window(const void* q, const void* kcache, const void* vcache, float* out,
                       int newTokens, int totalLen, int startPos, int Hq, int Hkv, int d_h, int B,
                       int window, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Bytes of device workspace attn_decode_paged needs (0 when it needs none).  The key
 * split is planned for the longest history the table can describe,
 * max_blocks * block_size.  Pure host arithmetic; 0 for arguments attn_decode_paged
 * would reject.
 */
size_t attn_decode_paged_workspace_bytes(int B, int newTokens, int Hq, int Hkv, int d_h,
                                         int block_size, int max_blocks, int dtype);

/*
 * Paged (block-table) cached decode: makarna's CausalAttentionPackedBlocks, and the
 * "paged decode attention" of Riftco's "Algorithm and cache boundaries" section (the
 * one-query inference algorithm reading a logical-to-physical K/V page table).  Per sequence b it computes
 * exactly attn_decode_cached over the history its blocks hold.
 *
 *   q, out          : [B, newTokens, Hq, d_h]  as in attn_decode_cached
 *   kpool, vpool    : [num_blocks, Hkv, block_size, d_h]  physical blocks; inside a block
 *                     the layout is head-major, [kvHead][tokenWithinBlock][headDim] (the
 *                     packed view layout)
 *   block_table     : [B, max_blocks] int32, DEVICE memory.  Logical block i of sequence b
 *                     (positions i*block_size .. i*block_size+block_size-1) is physical
 *                     block block_table[b*max_blocks + i].  Entries past the last block a
 *                     sequence needs are never read; blocks may be shared by sequences.
 *   seq_lens        : [B] int32, DEVICE memory.  History length of sequence b, new tokens
 *                     included: its new tokens sit at positions seq_lens[b]-newTokens ..
 *                     seq_lens[b]-1, and new token i attends to keys 0 .. seq_lens[b]-
 *                     newTokens+i.  Slots of a block past seq_lens[b] are never read.
 *   scale           : fixed at 1/sqrt(d_h)
 *   workspace       : at least attn_decode_paged_workspace_bytes(...) bytes
 *
 * Supported: dtype GQA_BF16 with d_h a multiple of 16 up to 128, block_size a positive
 * multiple of 16 (else GQA_EUNSUPPORTED).  Host-side errors as attn_decode_cached, plus
 * GQA_EINVAL for block_size, max_blocks or num_blocks <= 0 on a non-empty call,
 * max_blocks * block_size above 2^30, and NULL or misaligned table/lengths (4-byte
 * alignment).  The table and lengths live on the device and are checked by the kernels:
 * a sequence whose length is below newTokens or above max_blocks*block_size, or whose
 * needed table entries fall outside [0, num_blocks), gets NaN in all of its output
 * rows, and nothing outside the pools is read.
 */
int attn_decode_paged(const void* q, const void* kpool, const void* vpool,
                      const int* block_table, const int* seq_lens, float* out, int B,
                      int newTokens, int Hq, int Hkv, int d_h, int block_size, int max_blocks,
                      int num_blocks, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Cached decode over token-major KV blocks: makarna's CausalAttentionBlocks, whose views
 * each hold Length consecutive positions from Start on, K and V laid out token by token
 * with all KV heads of a token together ([t, Hkv*headDim]).  Here the views are the
 * blocks a block table names: logical block i of sequence b is the view with Start =
 * i*block_size and Length = min(block_size, seq_lens[b] - Start), so its key positions
 * are fixed by its place in the table.  Per sequence the result is exactly
 * attn_decode_paged (and attn_decode_cached) over the same history.
 *
 *   kpool, vpool    : [num_blocks, block_size, Hkv, d_h]  physical blocks, token-major
 *                     inside each block: [tokenWithinBlock][kvHead][headDim]
 *   everything else : as attn_decode_paged, workspace included
 *                     (attn_decode_paged_workspace_bytes(...) bytes)
 *
 * Supported shapes and every error case are those of attn_decode_paged.
 */
int attn_decode_blocks(const void* q, const void* kpool, const void* vpool,
                       const int* block_table, const int* seq_lens, float* out, int B,
                       int newTokens, int Hq, int Hkv, int d_h, int block_size, int max_blocks,
                       int num_blocks, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Local-window paged decode: attn_decode_paged where new token i of sequence b
 * (position seq_lens[b] - newTokens + i) sees only the last `window` positions up to
 * its own.  Table entries of blocks that lie entirely below the first new token's
 * window start (rounded down to a multiple of 32) are never read, so a sliding-window
 * cache may already have released them.  Arguments and errors as attn_decode_paged,
 * plus GQA_EINVAL for window < 1; the workspace is
 * attn_decode_paged_window_workspace_bytes(...).
 */
size_t attn_decode_paged_window_workspace_bytes(int B, int newTokens, int Hq, int Hkv, int d_h,
                                                int block_size, int max_blocks, int window,
                                                int dtype);
int attn_decode_paged_window(const void* q, const void* kpool, const void* vpool,
                             const int* block_table, const int* seq_lens, float* out, int B,
                             int newTokens, int Hq, int Hkv, int d_h, int block_size,
                             int max_blocks, int num_blocks, int window, int dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Prefill that also returns each row's softmax statistic, the input of attn_backward
 * (Riftco "Two exact full-sequence algorithms": the memory-linear path keeps per-row
 * statistics of shape [B, H, T] instead of the probabilities).  As attn_prefill (automatic
 * kernel choice, window 0), plus
 *   lse  [B, Hq, T] float32, 4-byte aligned: log sum_j exp(s_ij) over the row's visible
 *        keys, natural log, with s_ij = scale * <q_i, k_j> as in out; P_ij = exp(s_ij - lse_i).
 * The page keeps the row maximum and the exponential sum; their log-sum-exp carries the
 * same information in one number.  Errors as attn_prefill, plus GQA_EINVAL for a null or
 * misaligned lse.
 */
int attn_prefill_lse(const void* q, const void* k, const void* v, float* out, float* lse, int B, int Hq,
                     int Hkv, int T, int d_h, float scale, int causal, int dtype, void* stream);

/*
 * Backward pass of prefill (Riftco "Two exact full-sequence algorithms": recompute each
 * probability from Q, K and the row statistic, then apply the exact softmax
 * vector-Jacobian product).  Given the forward's inputs, its output `out`, its `lse`
 * (attn_prefill_lse) and the upstream gradient dout = dL/dout, writes the gradients of L:
 *   dq [B,Hq,T,d_h] = scale * sum_j dS_ij k_j
 *   dk [B,Hkv,T,d_h] = scale * sum over the group's query heads and rows of dS_ij q_i
 *   dv [B,Hkv,T,d_h] = sum over the group's query heads and rows of P_ij dout_i
 * with P_ij = exp(s_ij - lse_i), dS_ij = P_ij (dout_i . v_j - dout_i . out_i).
 *   q, k, v  of dtype, as the forward;  out, dout, lse, dq, dk, dv float32
 *   workspace: device memory of attn_backward_workspace_bytes(...) bytes, 256-byte aligned
 *   (two float32 statistics per row, and for the matrix-core path dout rounded to bf16)
 * bf16 with d_h a multiple of 16 up to 128 runs on the matrix cores; fp32 inputs and other
 * head dims up to 256 run on the vector ALU (fp32 throughout).  Errors as attn_prefill,
 * plus GQA_EWORKSPACE.  The result is deterministic (no atomics).
 */
size_t attn_backward_workspace_bytes(int B, int Hq, int Hkv, int T, int d_h, int dtype);
int attn_backward(const void* q, const void* k, const void* v, const float* out, const float* dout,
                  const float* lse, float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int T, int d_h,
                  float scale, int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * KV-cache append with NeoX rotary embedding on K: the step right before cached decode
 * (Hesper's attention layer, the fused RoPE-K + KV-cache-write kernels and their batched
 * prefill companion; the forge chapter's apply_rope at offset start_pos, then the cache
 * append).  New token i of sequence b, at absolute position p = start_pos + i, is written
 * to cache row p of every K/V head:
 *
 *   vcache[b,g,p,:] = v_new[b,i,g,:]
 *   kcache[b,g,p,j]       = k1 * cos(a_j) - k2 * sin(a_j)      for j < d_h/2, with
 *   kcache[b,g,p,j+d_h/2] = k2 * cos(a_j) + k1 * sin(a_j)      k1 = k_new[b,i,g,j],
 *                                                              k2 = k_new[b,i,g,j+d_h/2],
 *   a_j = p * rope_base^(-2j/d_h) / freq_factors[j]
 *
 * (the pages pair dim j with dim j + d_h/2 and name a base and per-pair frequency
 * factors; the angle above is the plain reading of that rotation).
 *   k_new, v_new   [B, newTokens, Hkv, d_h] float32, token-major (the projections' layout)
 *   kcache, vcache [B, Hkv, totalLen, d_h] of dtype; bf16 values are rounded to nearest
 *                  even from the float32 result.  Rows other than start_pos ..
 *                  start_pos+newTokens-1 are not touched.
 *   freq_factors   [d_h/2] float32 (4-byte aligned) or NULL for all ones; read only when
 *                  rope_base > 0
 *   rope_base      > 0 rotates K; 0 writes K unrotated
 * Angles are formed in double precision and reduced modulo 2*pi; the rotation is float32.
 * Errors: GQA_EINVAL for negative sizes, Hkv <= 0, start_pos + newTokens > totalLen, a
 * negative or non-finite rope_base, null or misaligned pointers; GQA_EUNSUPPORTED for d_h
 * not a multiple of 8 or above 256.
 */
int attn_kv_append(const float* k_new, const float* v_new, void* kcache, void* vcache,
                   const float* freq_factors, int B, int newTokens, int Hkv, int d_h, int totalLen,
                   int start_pos, float rope_base, int dtype, void* stream);

/*
 * The same append into paged pools [num_blocks, Hkv, block_size, d_h] (the layout of
 * attn_decode_paged): the new tokens of sequence b are its last newTokens positions,
 * p = seq_lens[b] - newTokens + i, stored in block block_table[b][p / block_size] at row
 * p % block_size.  block_table [B, max_blocks] and seq_lens [B] are int32 device arrays.
 * A sequence whose length is below newTokens or beyond max_blocks*block_size, or whose
 * needed table entry lies outside [0, num_blocks), is not written (the device-side
 * metadata cannot be checked before launch).  The blocks receiving new tokens must not be
 * shared between sequences (concurrent writes to one row race).  Other errors as
 * attn_kv_append, plus GQA_EINVAL for non-positive block_size, max_blocks or num_blocks.
 */
int attn_kv_append_paged(const float* k_new, const float* v_new, void* kpool, void* vpool,
                         const int* block_table, const int* seq_lens, const float* freq_factors,
                         int B, int newTokens, int Hkv, int d_h, int block_size, int max_blocks,
                         int num_blocks, float rope_base, int dtype, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
