/*
 * libattn -- exact scaled dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is caller-owned device memory (or NULL where a
 * parameter says it may be); the library allocates nothing and keeps no state
 * between calls.  Every call validates its arguments on the host before any HIP
 * call and, on error, returns a status without touching the stream.  On success
 * the work is enqueued asynchronously on `stream` (a hipStream_t passed as
 * void*; NULL means the null stream) and the call returns ATTN_OK once the
 * launches were accepted.  A launch failure reported by the HIP runtime returns
 * ATTN_ERR_HIP.  Calls are thread-safe.  Outputs must not alias inputs.
 *
 * Layouts are dense row-major:
 *   prefill  q, out [B, Hq, T, d_h];  k, v [B, Hkv, S, d_h];  lse [B, Hq, T] fp32
 *   decode   q, out [num_seqs, Hq, d_h];  k_cache, v_cache [num_blocks, Hkv, block_size, d_h]
 *            block_table [num_seqs, max_blocks_per_seq] int32;  seq_lens [num_seqs] int32;
 *            lse [num_seqs, Hq] fp32
 * out has the dtype of the inputs; accumulation and lse are fp32.
 * Alignment: tensors of head rows (q, k, v, out, their gradients, the caches, the gather's
 * destination and the workspaces) start on 16-byte boundaries, lse, block tables and
 * sequence lengths on 4-byte ones; otherwise the call returns ATTN_ERR_INVALID_ARG.
 */
#ifndef LIBATTN_ATTN_H
#define LIBATTN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_API __attribute__((visibility("default")))

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,  /* NULL pointer, non-positive size, Hq % Hkv != 0, bad table size */
  ATTN_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement (d_h, dtype, block_size) */
  ATTN_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than the *_workspace_bytes() size */
  ATTN_ERR_HIP = 4,          /* the HIP runtime rejected a launch */
  ATTN_ERR_SCRATCH = 5       /* request larger than the static scratch of attn_decode_paged_static */
} attn_status_t;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype_t;

/*
 * attn_fwd -- exact attention softmax(Q K^T / sqrt(d_h)) V over whole sequences
 * ("22 interview questions on attention & transformers", How does self-attention
 * work; "Transformer Attention Mechanism Interview Deep Dive", Scaled dot-product
 * attention), computed with the blocked online softmax of "Why is attention O(n^2),
 * how does FlashAttention help ..." (Deep dive: FlashAttention): the T x S score
 * matrix is never written to memory.
 *
 *   q        [B, Hq, T, d_h]   queries, dtype `dtype`
 *   k, v     [B, Hkv, S, d_h]  keys and values; query head h reads KV head
 *                              h / (Hq / Hkv) (grouped-query sharing, contiguous groups)
 *   out      [B, Hq, T, d_h]   result, dtype `dtype`
 *   lse      [B, Hq, T] fp32 or NULL: natural log of the sum over visible keys of
 *                              exp(q.k / sqrt(d_h)) (the saved statistic a backward
 *                              pass recomputes probabilities from); -inf for a row
 *                              with no visible key
 *   causal   0 or 1: key s is visible to query row t iff s <= pos + t; hidden logits
 *            are -inf before the softmax ("Causal masking" of the Deep Dive page), and
 *            key blocks hidden from every row of a query block are skipped
 *   rope_base  > 0: rotate q and k at load, adjacent pairs (2i, 2i+1) by the angle
 *            position * rope_base^(-2i/d_h) ("How does Rotary Position Embedding (RoPE)
 *            work?"); query row t sits at position pos + t, key s at position s.
 *            0 disables the rotation.
 *   pos      absolute position of query row 0 (0 for self-attention over a prompt)
 *   workspace, workspace_bytes  optional device scratch (16-byte aligned), caller-owned, no
 *            clearing needed; overlapping calls must not share one.  With bf16, RoPE and at
 *            least B * Hkv * S * d_h * 2 bytes, k is rotated once into it by a first kernel
 *            and the prefill reads that copy; otherwise (NULL, smaller, fp32 or no RoPE) each
 *            key block is rotated as it lands in the prefill, once per query block that reads
 *            it.  attn_fwd_workspace_bytes says when the first pays.  Same definition either
 *            way; the rotated keys are rounded to bf16 from slightly different angle
 *            arithmetic, so the two results may differ in the last bits.
 *   dtype    ATTN_F32 or ATTN_BF16 (bf16 inputs use bf16 MFMA with fp32 accumulation)
 *
 * Supported: d_h in {64, 128}; any B, Hq, Hkv >= 1 with Hq % Hkv == 0; any
 * T, S >= 1 (ragged tails are masked) with S * d_h * 2 < 2^32 for bf16 (one KV head's
 * keys are addressed through a 32-bit buffer range; ATTN_ERR_UNSUPPORTED otherwise).
 * The 1/sqrt(d_h) scale is fixed.
 */
ATTN_API attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                       int B, int Hq, int Hkv, int T, int S, int d_h, int causal,
                       float rope_base, int64_t pos, void* workspace, size_t workspace_bytes,
                       attn_dtype_t dtype, void* stream);

/*
 * Bytes of workspace worth giving attn_fwd (window 0) or attn_fwd_window (window >= 1)
 * for these sizes: B * Hkv * S * d_h * 2 when the keys are better rotated once ahead of the
 * prefill (bf16 with RoPE, and each key block read by at least 16 of the prefill's
 * workgroups of 256 query rows, so that the extra pass over k costs less than the repeated
 * rotation); 0 when not, or on invalid sizes.
 */
ATTN_API size_t attn_fwd_workspace_bytes(int B, int Hq, int Hkv, int T, int S, int d_h, int causal,
                                         int64_t window, float rope_base, int64_t pos,
                                         attn_dtype_t dtype);

/*
 * attn_fwd_window -- causal sliding-window attention: key s is visible to query row t
 * iff pos + t - window < s <= pos + t, i.e. each query sees the `window` most recent
 * positions up to its own ("22 interview questions on attention & transformers", What
 * is sparse / sliding-window attention: each token attends to a fixed neighbourhood of
 * size w, cost O(n w); "Why is attention O(n^2) ...", Long context in practice: sliding
 * window of width w, O(T w)).  Key blocks outside the window are not visited.
 *
 * Arguments, layouts, RoPE, the workspace and the result are as for attn_fwd with
 * causal = 1; window >= 1 (ATTN_ERR_INVALID_ARG otherwise), and a window reaching back past
 * key 0 gives exactly the causal result.
 */
ATTN_API attn_status_t attn_fwd_window(const void* q, const void* k, const void* v, void* out,
                                       float* lse, int B, int Hq, int Hkv, int T, int S, int d_h,
                                       int64_t window, float rope_base, int64_t pos,
                                       void* workspace, size_t workspace_bytes,
                                       attn_dtype_t dtype, void* stream);

/*
 * attn_fwd_fp8 -- exact attention with fp8 inputs and fp8 matrix products ("Why is attention
 * O(n^2), how does FlashAttention help ...", Deep dive: later FlashAttention versions exploit
 * newer hardware such as FP8), same definition and masking as attn_fwd.
 *
 *   q8       [B, Hq, T, d_h]   E4M3 codes (OCP 8-bit float: bias 7, largest 448, no infinity)
 *   k8       [B, Hkv, S, d_h]  E4M3 codes
 *   vt8      [B, Hkv, d_h, S]  E4M3 codes of V, transposed (d_h-major), 4-byte aligned
 *   q_scale, k_scale, v_scale  > 0: the value of a code c of that tensor is c * scale
 *   out      [B, Hq, T, d_h] bf16;  lse [B, Hq, T] fp32 or NULL (as attn_fwd)
 *   causal, pos  as attn_fwd.  q and k are used as given (already rotated: no RoPE).
 * Both products run on E4M3 matrix cores with fp32 accumulation; the probabilities are
 * rounded to E4M3 for the P V product, the softmax normaliser uses them unrounded.
 * Supported: d_h == 128, S % 4 == 0 (ATTN_ERR_UNSUPPORTED otherwise); codes must not be NaN.
 */
ATTN_API attn_status_t attn_fwd_fp8(const void* q8, const void* k8, const void* vt8, void* out,
                                    float* lse, int B, int Hq, int Hkv, int T, int S, int d_h,
                                    int causal, float q_scale, float k_scale, float v_scale,
                                    int64_t pos, void* stream);

/*
 * attn_decode_paged -- one decode step over a block-tabled KV cache ("Self-Attention
 * Complexity, FlashAttention, PagedAttention, and RoPE in Code", Part 3: fixed-size
 * blocks and per-sequence block tables; "Why is attention O(n^2) ...": a decode step
 * attends to every cached key and is memory-bound).
 *
 *   q            [num_seqs, Hq, d_h]  the one new query token of each sequence; it is
 *                rotated at position seq_lens[b] - 1 when rope_base > 0
 *   k_cache, v_cache  [num_blocks, Hkv, block_size, d_h]  physical block pool; cached K
 *                is used as stored (already rotated at its own position)
 *   block_table  [num_seqs, max_blocks_per_seq] int32: token j of sequence b lives in
 *                slot j % block_size of physical block block_table[b][j / block_size];
 *                entries past the sequence are ignored
 *   seq_lens     [num_seqs] int32: cached tokens per sequence (current one included);
 *                device contract: 1 <= seq_lens[b] <= max_blocks_per_seq * block_size and
 *                every used table entry in [0, num_blocks) (entries outside are clamped into
 *                the pool: no fault, but that sequence's result is undefined)
 *   out          [num_seqs, Hq, d_h] dtype `dtype`;  lse [num_seqs, Hq] fp32 or NULL
 *   workspace    device scratch of at least attn_decode_workspace_bytes(...) bytes for
 *                the partial results; caller-owned, contents need no clearing; two calls
 *                that overlap in time must not share one workspace
 *   dtype        ATTN_BF16 only (ATTN_F32 returns ATTN_ERR_UNSUPPORTED)
 *
 * Supported: block_size == 16, d_h == 128, Hq % Hkv == 0, Hq / Hkv <= 16,
 * num_seqs * Hkv * max_blocks_per_seq <= 2^30.
 * All (sequence, KV head, block) triples are cut into equal runs read in parallel
 * (split-K along the key axis, balanced whatever the length mix); a second kernel
 * merges the partial (output, max, normaliser) triples with a log-sum-exp merge.
 */
ATTN_API attn_status_t attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int block_size, int num_seqs, int Hq, int Hkv, int d_h,
                                int max_blocks_per_seq, int num_blocks, float rope_base,
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                attn_dtype_t dtype, void* stream);

/* Bytes of device scratch attn_decode_paged_static holds per GPU (32 MiB). */
#define ATTN_DECODE_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * attn_decode_paged_static -- attn_decode_paged with no workspace argument that allocates
 * nothing, for callers that cannot allocate device memory: code under HIP graph capture,
 * serving loops that must not enter an allocator, harnesses that forbid allocation.
 *
 * The partial results that attn_decode_paged keeps in the caller's workspace live instead in
 * a device array of ATTN_DECODE_STATIC_SCRATCH_BYTES inside the library, one per GPU, held
 * until the process ends; its address is looked up (hipGetSymbolAddress) on the first call
 * on each GPU.  A request for which attn_decode_workspace_bytes(...) exceeds that size
 * returns ATTN_ERR_SCRATCH before anything is launched (e.g. with Hq / Hkv = 4 it fits up to
 * num_seqs * Hkv = 14000; with Hq / Hkv = 16 up to 1900).  Arguments, checks, errors and
 * results are otherwise those of attn_decode_paged, and the outputs are bit-identical to it.
 * All calls on one GPU share that GPU's array, which keeps the last call's contents (the
 * kernels need it in no particular state): calls that overlap in time on one GPU, from two
 * streams or two host threads, race, and the caller must order them.  The call makes no
 * hipMalloc, hipFree or other allocating request.
 */
ATTN_API attn_status_t attn_decode_paged_static(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int block_size, int num_seqs, int Hq, int Hkv, int d_h,
                                int max_blocks_per_seq, int num_blocks, float rope_base,
                                void* out, float* lse, attn_dtype_t dtype, void* stream);

/*
 * attn_prefill_paged -- prefill (or chunked prefill) of T new query tokens per sequence
 * whose keys and values, including any shared prefix, sit in a block-tabled cache
 * ("Self-Attention Complexity, FlashAttention, PagedAttention, and RoPE in Code", Part 3:
 * fixed-size blocks, per-sequence block tables, and blocks shared between sequences that
 * have a common prefix).  Several block tables may name the same physical blocks; the
 * kernel only reads the cache.
 *
 *   q            [num_seqs, Hq, T, d_h]: the last T tokens of each sequence; query row t of
 *                sequence b sits at position seq_lens[b] - T + t and is rotated there when
 *                rope_base > 0
 *   k_cache, v_cache, block_table, seq_lens, block_size, max_blocks_per_seq, num_blocks
 *                as for attn_decode_paged (cached K already rotated; seq_lens[b] counts the
 *                new tokens, whose K and V the caller has written into the cache)
 *   out          [num_seqs, Hq, T, d_h] bf16;  lse [num_seqs, Hq, T] fp32 or NULL
 * Key s is visible to query row t iff s <= seq_lens[b] - T + t (causal over the whole
 * sequence).  Device contract: T <= seq_lens[b] <= max_blocks_per_seq * block_size (rows
 * whose position is negative get output 0 and lse -inf); table entries outside
 * [0, num_blocks) are clamped into the pool (no fault; such a sequence's result is
 * undefined).
 * Supported: bf16, d_h == 128, block_size == 16, max_blocks_per_seq <= 4096, Hq % Hkv == 0.
 */
ATTN_API attn_status_t attn_prefill_paged(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          int block_size, int num_seqs, int Hq, int Hkv, int d_h,
                                          int T, int max_blocks_per_seq, int num_blocks,
                                          float rope_base, void* out, float* lse, attn_dtype_t dtype,
                                          void* stream);

/*
 * attn_bwd -- gradients of exact attention (as computed by attn_fwd / attn_fwd_window)
 * with respect to q, k and v.  The probabilities are recomputed from the forward's saved
 * lse instead of being stored ("Why is attention O(n^2), how does FlashAttention help
 * ...", Deep dive: FlashAttention; "Self-Attention Complexity, FlashAttention,
 * PagedAttention, and RoPE in Code", Part 2); the gradients themselves follow from the
 * chain rule: dV = P^T dO, dS = P * (dO V^T - rowsum(dO * O)), dq' = dS k' / sqrt(d_h),
 * dk' = dS^T q' / sqrt(d_h), with q', k' the rotated inputs and dq, dk rotated back.
 *
 *   q, k, v, causal, window, rope_base, pos   as given to the forward call (window 0: no
 *            window; window >= 1 requires causal = 1)
 *   out      [B, Hq, T, d_h] the forward's output;  lse [B, Hq, T] fp32 the forward's lse
 *   dout     [B, Hq, T, d_h] gradient of the loss with respect to out
 *   dq       [B, Hq, T, d_h];  dk, dv [B, Hkv, S, d_h]: results (dtype of the inputs).  With
 *            grouped-query attention dk and dv of a KV head sum over the query heads that
 *            read it.  Keys no query sees get zero gradients.
 *   workspace  device scratch of at least attn_bwd_workspace_bytes(...) bytes (per-row
 *            statistics and, with RoPE, the rotated q and k); caller-owned, no clearing
 *            needed; overlapping calls must not share one workspace
 * Supported: bf16, d_h == 128 (ATTN_ERR_UNSUPPORTED otherwise).  Three kernels are
 * enqueued on `stream`; results are deterministic (no atomics).
 */
ATTN_API attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* out,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                int B, int Hq, int Hkv, int T, int S, int d_h, int causal,
                                int64_t window, float rope_base, int64_t pos, void* workspace,
                                size_t workspace_bytes, attn_dtype_t dtype, void* stream);

/* Bytes of workspace attn_bwd needs for these sizes (0 on invalid sizes). */
ATTN_API size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int T, int S, int d_h,
                                         float rope_base);

/* Bytes of workspace attn_decode_paged needs for these sizes (0 on invalid sizes). */
ATTN_API size_t attn_decode_workspace_bytes(int num_seqs, int Hq, int Hkv, int d_h,
                                   int max_blocks_per_seq, int block_size);

/*
 * attn_paged_gather -- copy each sequence's cached rows into a contiguous buffer through the
 * read path of attn_decode_paged itself: the same work division, block-table reads (64
 * entries at a time, broadcast across the wave), slice addresses (table entries clamped into
 * [0, num_blocks)) and LDS staging, with the attention replaced by a copy.  It exists so that
 * the decode's block-table translation ("Self-Attention Complexity, FlashAttention,
 * PagedAttention, and RoPE in Code", Part 3) can be checked bit for bit.
 *
 *   cache        [num_blocks, Hkv, block_size, d_h] elements of elem_bytes (2 or 4), 16-byte aligned
 *   dst          [num_seqs, Hkv, max_blocks_per_seq * block_size, d_h], 16-byte aligned; rows
 *                j >= seq_lens[b] are left untouched
 * Supported: block_size == 16 and d_h * elem_bytes == 256 (the decode cache's rows: bf16,
 * d_h = 128), num_seqs * Hkv * max_blocks_per_seq <= 2^30 (ATTN_ERR_UNSUPPORTED otherwise).
 */
ATTN_API attn_status_t attn_paged_gather(const void* cache, const int32_t* block_table,
                                const int32_t* seq_lens, int block_size, int num_seqs, int Hkv,
                                int d_h, int max_blocks_per_seq, int num_blocks, int elem_bytes,
                                void* dst, void* stream);

/* Static description of a status code. */
ATTN_API const char* attn_status_str(attn_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_ATTN_H */
