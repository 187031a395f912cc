/*
 * attn.h — C ABI of libattn.so: causal grouped-query attention forward with
 * rotary embeddings and ALiBi for AMD Instinct MI355X (gfx950).
 *
 * The operation (fixed by the source pages):
 *   out[b,h,i] = sum_j softmax_j( <R(p_i) q[b,h,i], R(p_j) k[b,g,j]> / sqrt(hd)
 *                                 - slope_h * |i - j| ) * v[b,g,j]
 *   with g = h / (H / KV) (grouped-query sharing, consecutive groups),
 *   j <= i when causal, R(p) the interleaved-pair rotary rotation at position p
 *   (pair (2m, 2m+1) turned by p * base^(-2m/hd)), V never rotated.
 *   Sources: "Building a Transformer from Scratch: Attention, Architecture, and
 *   Memory" (Part 1, scaled dot-product equation; Part 3, the online-softmax
 *   recurrences), "Write attention from scratch" (the lab listing: rope with a
 *   position offset, np.repeat grouping, lower-triangular mask), "Building a
 *   Multi-Head Self-Attention Block with RoPE and ALiBi from Scratch" (Step 3:
 *   ALiBi bias as slope times distance, added after the 1/sqrt(d_k) scaling),
 *   "Building Grouped-Query Attention with RoPE and Flash Attention from
 *   Scratch" (Step 3: tiled online softmax; roadmap: bf16 inputs with fp32
 *   softmax statistics and accumulation; cache written by position).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never frees, retains or allocates memory and never synchronises.
 *   - Tensors are dense, row-major, with the shapes stated per function.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     runs asynchronously; a return of ATTN_OK means "enqueued".
 *   - Every argument is validated before any HIP call; on failure nothing is
 *     enqueued, the status code says why and attn_last_error() gives detail.
 *   - No C++ exception crosses this boundary. Functions are thread-safe; the
 *     error text is per calling thread.
 *   - dtype / out_dtype: ATTN_DTYPE_F32 or ATTN_DTYPE_BF16. Softmax statistics
 *     and accumulation are always fp32; bf16 outputs are rounded to nearest
 *     even.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 5

/* Status codes. */
#define ATTN_OK 0
#define ATTN_ERR_NULL 1        /* a required pointer is NULL */
#define ATTN_ERR_SHAPE 2       /* non-positive size, H % KV != 0, odd hd, negative pos0, size overflow */
#define ATTN_ERR_UNSUPPORTED 3 /* hd not in {8,16,32,64,128}, unknown dtype / flag value */
#define ATTN_ERR_ALIGN 4       /* q/k/v/out/cache pointers not 16-byte aligned, workspace not 256-byte aligned */
#define ATTN_ERR_WORKSPACE 5   /* workspace missing or smaller than the *_workspace_bytes() figure */
#define ATTN_ERR_HIP 6         /* a HIP launch failed (no device, invalid stream, ...) */

/* Element types. */
#define ATTN_DTYPE_F32 0
#define ATTN_DTYPE_BF16 1

/* ALiBi slope families (the bias itself is -slope_h * |i - j|). */
#define ATTN_ALIBI_NONE 0
#define ATTN_ALIBI_GEOMETRIC 1 /* slope_h = 2^(-8(h+1)/H), h = 0..H-1 */
#define ATTN_ALIBI_PAGE1 2     /* slope_h = 2^(-2(h+1)/H): the heuristic printed in Step 1 of the
                                  multi-head RoPE+ALiBi page */

/* ABI version of the loaded library (ATTN_ABI_VERSION it was built with). */
int attn_abi_version(void);

/* Static, never-NULL name of a status code ("ATTN_OK", ..., "unknown status"). */
const char* attn_status_str(int status);

/* Detail of the last non-OK status returned to this thread ("" if none). */
const char* attn_last_error(void);

/*
 * Timing hook for benchmarks and profilers. `start` and `stop` are hipEvent_t
 * handles created by the caller (or NULL to clear). The next prefill, decode
 * or backward call made by the same thread records `start` on its stream
 * immediately before launching its main kernel (the attention kernel of
 * prefill, the split-KV kernel of decode, the dq and dk/dv kernels of the
 * backward) and `stop` immediately after it, then clears the hook. The events stay owned by the caller. Always returns ATTN_OK.
 */
int attn_set_timing_events(void* start, void* stop);

/*
 * Bytes of device workspace attn_prefill_fwd needs: the rotated keys,
 * B*KV*T*hd elements of `dtype`, when rope_base != 0; 0 without rotary
 * embedding. Returns 0 for invalid sizes (the forward call reports why).
 */
size_t attn_prefill_workspace_bytes(int B, int T, int KV, int hd, int dtype, double rope_base);

/*
 * Prefill / full-sequence attention forward ("Building Grouped-Query Attention
 * with RoPE and Flash Attention from Scratch", Step 3, with the causal mask of
 * "Write attention from scratch" and ALiBi of the multi-head page, Step 3).
 *
 *   q    [B, H,  T, hd]  dtype, before rotation
 *   k    [B, KV, T, hd]  dtype, before rotation
 *   v    [B, KV, T, hd]  dtype
 *   out  [B, H,  T, hd]  out_dtype (written)
 *   lse  [B, H,  T]      fp32 natural-log log-sum-exp of each row's scaled,
 *                        biased scores (written); may be NULL
 *   Token t of every sequence sits at position pos0 + t (for the rotation);
 *   the causal test and the ALiBi distance use token indices.
 *   rope_base: rotary base (10000, 500000, ...); 0 disables the rotation.
 *   causal: 1 keeps keys j <= i, 0 attends all keys.
 *   alibi: ATTN_ALIBI_* (0 = none).
 *   Scale is fixed at 1/sqrt(hd).
 *   workspace: device scratch of at least attn_prefill_workspace_bytes(...)
 *   bytes (may be NULL when that figure is 0); its contents are clobbered.
 *
 * q, k, v, out and workspace must not overlap. bf16 inputs with hd in
 * {64,128} run on the matrix-core (MFMA) kernel; every other supported case
 * runs on a vector-ALU kernel with fp32 arithmetic throughout.
 */
int attn_prefill_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     int B, int T, int H, int KV, int hd, int pos0, double rope_base,
                     int causal, int alibi, int dtype, int out_dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunked prefill and sliding-window attention: the same forward for a chunk
 * of Tq queries that are tokens q_offset .. q_offset+Tq-1 of a Tk-token key
 * sequence (a prompt processed chunk by chunk, as lab Exercise 2 of "Write
 * attention from scratch" does token by token), optionally restricted to a
 * sliding window of the last `window` tokens (that page's Exercise 3; the
 * sliding-window mode on the roadmap of "Building Grouped-Query Attention with
 * RoPE and Flash Attention from Scratch").
 *
 *   q    [B, H,  Tq, hd]  dtype, before rotation; row i is token q_offset + i
 *   k    [B, KV, Tk, hd]  dtype, before rotation (the chunk's own keys are
 *                         tokens q_offset .. q_offset+Tq-1 of it)
 *   v    [B, KV, Tk, hd]  dtype
 *   out  [B, H,  Tq, hd]  out_dtype (written)
 *   lse  [B, H,  Tq]      fp32 (written); may be NULL
 *   Key token j sits at position pos0 + j, query row i at pos0 + q_offset + i.
 *   causal: 1 keeps keys j <= q_offset + i. window > 0 (causal only) keeps
 *   only keys j > q_offset + i - window, i.e. the query's own token and the
 *   window - 1 before it; 0 means no window. ALiBi distances are in tokens.
 *   workspace: at least attn_prefill_workspace_bytes(B, Tk, KV, hd, dtype,
 *   rope_base) bytes.
 *
 * Requires 0 <= q_offset and q_offset + Tq <= Tk (ATTN_ERR_SHAPE otherwise);
 * window < 0 is ATTN_ERR_SHAPE, window > 0 with causal = 0 ATTN_ERR_UNSUPPORTED.
 * Keys outside every query's window must still hold finite values (their
 * zero weights multiply them). attn_prefill_fwd is this call with
 * Tq = Tk = T, q_offset = 0, window = 0. Other rules as attn_prefill_fwd.
 */
int attn_prefill_ex_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                        int B, int Tq, int Tk, int H, int KV, int hd, int pos0, int q_offset,
                        int window, double rope_base, int causal, int alibi, int dtype,
                        int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace attn_prefill_bwd needs: rotated copies of K and Q
 * (only when rope_base != 0) and one fp32 per query row. 0 for invalid sizes.
 */
size_t attn_prefill_bwd_workspace_bytes(int B, int T, int H, int KV, int hd, int dtype, double rope_base);

/*
 * Backward of attn_prefill_fwd: the gradients of sum(out * dout) with respect
 * to the pre-rotation q, k and v (the derivative of the softmax attention of
 * "Building Grouped-Query Attention with RoPE and Flash Attention from
 * Scratch", Step 3, whose backward the multi-head page's gradient-flow test and
 * the pure-Python page's finite-difference test exercise). The attention
 * weights are recomputed from q, k and the forward's lse (never stored):
 *   dv_j = sum_i p_ij dout_i,  ds_ij = p_ij (<dout_i, v_j> - <dout_i, out_i>),
 *   dq = R(-pos) scale sum_j ds_ij k'_j,  dk = R(-pos) scale sum_i ds_ij q'_i,
 * with k', q' rotated; GQA sums dk, dv over the group's query heads.
 *
 *   q, k, v    as for attn_prefill_fwd (dtype, pre-rotation)
 *   out        [B, H, T, hd]  the forward's output (out_dtype)
 *   lse        [B, H, T]      the forward's fp32 log-sum-exp (required)
 *   dout       [B, H, T, hd]  gradient of the loss w.r.t. out (out_dtype)
 *   dq         [B, H, T, hd]  grad_dtype (written)
 *   dk, dv     [B, KV, T, hd] grad_dtype (written, not accumulated)
 *   pos0, rope_base, causal, alibi as in the forward call.
 *   workspace: at least attn_prefill_bwd_workspace_bytes(...) bytes.
 *
 * Same validation rules and codes as attn_prefill_fwd; grad_dtype in {F32,
 * BF16}. bf16 inputs with hd in {64,128} run on matrix-core kernels; every
 * other supported case on vector-ALU kernels with fp32 arithmetic.
 */
int attn_prefill_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int T, int H, int KV, int hd,
                     int pos0, double rope_base, int causal, int alibi, int dtype, int out_dtype,
                     int grad_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace attn_decode_fwd needs for its split-KV partials
 * (fp32 partial outputs and their max / denominator per split). 0 for invalid
 * sizes.
 */
size_t attn_decode_workspace_bytes(int B, int H, int KV, int hd, int Lmax);

/*
 * One KV-cache decode step for B sequences ("Write attention from scratch",
 * Exercise 2: the incremental result equals the full computation; "Building
 * Grouped-Query Attention ...", roadmap: a pre-allocated cache written by
 * position; "Building a Transformer from Scratch", Part 3: KV caching).
 *
 *   q          [B, H,  hd]        dtype, the new token's query before rotation
 *   k_new      [B, KV, hd]        dtype, the new token's key before rotation
 *   v_new      [B, KV, hd]        dtype
 *   k_cache    [B, KV, Lmax, hd]  dtype, rotated keys at slots 0..L-1 (read);
 *                                 slot L receives R(L) k_new (written)
 *   v_cache    [B, KV, Lmax, hd]  dtype, values at slots 0..L-1 (read);
 *                                 slot L receives v_new (written)
 *   cache_lens [B] int32 device   L = cache_lens[b] >= 0 tokens already cached;
 *                                 must satisfy L < Lmax. The host does not read
 *                                 device memory, so this is checked on the
 *                                 device: a sequence with L outside [0, Lmax)
 *                                 gets NaN in out and lse and its cache rows
 *                                 are neither read nor written.
 *   out        [B, H, hd]         out_dtype (written)
 *   lse        [B, H]             fp32 (written); may be NULL
 *   The new token sits at position L: its query and key are rotated at L and
 *   the query attends slots 0..L inclusive (ALiBi distance L - j).
 *   workspace: at least attn_decode_workspace_bytes(B, H, KV, hd, Lmax) bytes.
 *   Lmax may be at most 2^24 (16,777,216) slots (ATTN_ERR_SHAPE otherwise);
 *   a (sequence, head) slab of the cache may exceed 2 GiB.
 *
 * k_new and v_new may both be NULL: slot L of every sequence then already
 * holds the new token's key (rotated) and value, as attn_qkv_proj_cache_fwd
 * leaves them, and nothing is written to the caches. rope_base still applies
 * to q; pass 0 when q comes rotated from that projection.
 *
 * Runs, in stream order: the cache append, the split-KV partial kernel, and
 * the log-sum-exp merge of the partials.
 */
int attn_decode_fwd(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const int32_t* cache_lens, void* out, float* lse,
                    int B, int H, int KV, int hd, int Lmax, double rope_base, int alibi,
                    int dtype, int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc. Arguments, results and kernels are those of
 * attn_decode_fwd (outputs bitwise equal). The split partials live in a
 * library-owned static device array of 32 MiB per GPU (created when the
 * library's code is loaded on that GPU, held until the process ends); the
 * stream must belong to the current device. The partials of one step take
 * B * H * ceil(Lmax / split) * (hd * 4 + 8) bytes, rounded up to 256, where
 * split is 256 slots on the vector-ALU path and 512 or 1024 on the
 * matrix-core path (1024 when B * KV * ceil(Lmax / 1024) >= 1024); a step that
 * needs more returns ATTN_ERR_WORKSPACE before any HIP call. (The 64-sequence,
 * 8193-slot, 32-head, hd-128 step needs 8.5 MB.) Nothing is allocated, freed
 * or cleared: every partial the merge reads is written first in the same
 * call. Calls that overlap in time on one GPU (different streams or host
 * threads) share the array and race; serialise them.
 */
int attn_decode_fwd_noalloc(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* cache_lens, void* out, float* lse,
                            int B, int H, int KV, int hd, int Lmax, double rope_base, int alibi,
                            int dtype, int out_dtype, void* stream);

/*
 * The same decode step over a cache held in 8-bit floats, the quantized
 * storage that "Build a Transformer Self-Attention Block from Scratch in Pure
 * Python" lists on its roadmap against the memory-bandwidth bottleneck (the
 * pages fix no format). Each cache element is an OCP FP8 E4M3 code (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits; subnormals; no infinities;
 * largest finite magnitude 448) standing for code_value * scale, with one
 * scale for all of K and one for all of V.
 *
 *   k_cache, v_cache  [B, KV, Lmax, hd] uint8 E4M3 codes: rotated keys / values
 *                     at slots 0..L-1 (read); slot L receives the codes of
 *                     R(L) k_new / k_scale and v_new / v_scale (written): the
 *                     value is clamped to +-448 and rounded to nearest, ties to
 *                     even mantissa, sign bit copied.
 *   k_scale, v_scale  positive finite fp32 scales.
 *   q, k_new, v_new   bf16 (dtype must be ATTN_DTYPE_BF16); every other
 *                     argument as for attn_decode_fwd (same workspace size).
 * The query attends slots 0..L of the dequantized cache, the new slot as
 * stored. Supported: hd in {64, 128}, H / KV <= 16 (ATTN_ERR_UNSUPPORTED
 * otherwise; ATTN_ERR_SHAPE for a non-positive or non-finite scale). Traffic
 * per step is half that of a bf16 cache.
 */
int attn_decode_fp8_fwd(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                        const int32_t* cache_lens, void* out, float* lse,
                        int B, int H, int KV, int hd, int Lmax, double rope_base, int alibi,
                        float k_scale, float v_scale, int dtype, int out_dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace attn_decode_latent_fwd needs (folded queries,
 * split partials, merged latent outputs, the split kernel's work list); 0 for
 * non-positive sizes.
 */
size_t attn_decode_latent_workspace_bytes(int B, int H, int dc, int Lmax);

/*
 * One decode step with a latent cache ("Write attention from scratch",
 * Exercise 5: keys and values are per-head up-projections of one short latent
 * per token, and the key up-projection folds into the query). With the
 * latent c_j of token j, head h's key is c_j W_uk[h] and its value c_j W_uv[h]:
 *   s_hj = <q_h, c_j W_uk[h]> / sqrt(hd) (+ ALiBi bias -slope_h (L - j))
 *        = <W_uk[h] q_h, c_j> / sqrt(hd),   out_h = (sum_j p_hj c_j) W_uv[h].
 * No rotary embedding on this path (a rotation of the keys would not commute
 * with the fold).
 *
 *   q          [B, H, hd]       bf16, the new token's queries
 *   c_new      [B, dc]          bf16, its latent
 *   c_cache    [B, Lmax, dc]    bf16, latents at slots 0..L-1 (read); slot L
 *                               receives c_new (written)
 *   cache_lens [B] int32 device L = cache_lens[b]; a sequence with L outside
 *                               [0, Lmax) gets NaN and its cache is untouched
 *   w_uk, w_uv [H, dc, hd]      bf16 up-projections (row c of W[h] maps latent
 *                               dim c to the head's hd dims)
 *   out        [B, H, hd]       out_dtype (written)
 *   lse        [B, H]           fp32 (written; may be NULL), log-sum-exp of the
 *                               scores over slots 0..L
 *   workspace  at least attn_decode_latent_workspace_bytes(B, H, dc, Lmax)
 * Supported: dtype ATTN_DTYPE_BF16, hd in {64, 128}, dc in {256, 512}, any H.
 * Runs, in stream order: the query fold, the split-KV attention over the
 * latent cache (which appends c_new), the merge and the value up-projection.
 */
int attn_decode_latent_fwd(const void* q, const void* c_new, void* c_cache, const int32_t* cache_lens,
                           const void* w_uk, const void* w_uv, void* out, float* lse,
                           int B, int H, int hd, int dc, int Lmax, int alibi, int dtype, int out_dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused QKV input projection with rotary embedding ("Building Grouped-Query
 * Attention with RoPE and Flash Attention from Scratch", Architecture Overview
 * and Step 4: one projection of x emits q, k and v with fewer K/V heads than
 * query heads, then q and k are rotated).
 *
 *   x      [B, T, D]            bf16, token t of sequence b
 *   w_qkv  [(H + 2 KV) hd, D]   bf16: the rows of W_q (H hd), then W_k (KV hd),
 *                               then W_v (KV hd), each an nn.Linear weight
 *                               [out, in], so the projection is x w_qkv^T
 *   q      [B, H,  T, hd]       bf16 (written), rotated at position pos0 + t
 *   k      [B, KV, T, hd]       bf16 (written), rotated at position pos0 + t
 *   v      [B, KV, T, hd]       bf16 (written)
 *   rope_base: rotary base; 0 disables the rotation (interleaved pairs, the
 *   same convention as attn_prefill_fwd, so q and k from here feed it with
 *   rope_base 0).
 * The products accumulate in fp32 on the matrix cores; the rotation is applied
 * to the fp32 sums, which are then rounded once to bf16.
 * Supported: dtype ATTN_DTYPE_BF16, hd in {64, 128}, D a multiple of 64 and
 * every operand under 2 GiB (ATTN_ERR_UNSUPPORTED / ATTN_ERR_SHAPE otherwise).
 * Pointers 16-byte aligned; x, w_qkv and the outputs must not overlap.
 */
int attn_qkv_proj_fwd(const void* x, const void* w_qkv, void* q, void* k, void* v,
                      int B, int T, int D, int H, int KV, int hd, int pos0, double rope_base,
                      int dtype, void* stream);

/*
 * The same projection for tokens appended to a KV cache (a decode step with
 * T = 1, or a prompt chunk; the pre-allocated cache written by position of the
 * GQA page's roadmap and lab Exercise 2 of "Write attention from scratch"):
 * token t of sequence b sits at position L + t, L = cache_lens[b], and its
 * rotated key and its value are written to slot L + t of k_cache / v_cache
 * [B, KV, Lmax, hd] (bf16). q [B, H, T, hd] as above. A sequence with L < 0 or
 * L + T > Lmax (checked on the device) gets NaN queries and its cache rows
 * are not written. cache_lens is not modified. Other rules as
 * attn_qkv_proj_fwd; requires 1 <= T <= Lmax.
 */
int attn_qkv_proj_cache_fwd(const void* x, const void* w_qkv, void* q, void* k_cache, void* v_cache,
                            const int32_t* cache_lens, int B, int T, int D, int H, int KV, int hd, int Lmax,
                            double rope_base, int dtype, void* stream);

/*
 * Output projection (the GQA page's Step 4: the attention output is
 * transposed back to [B, T, H hd] and mixed by o_proj):
 *   o    [B, H, T, hd]   bf16, the attention output
 *   w_o  [D, H hd]       bf16, nn.Linear weight
 *   y    [B, T, D]       out_dtype (written): y[b, t] = concat_h o[b, h, t] w_o^T
 * The transpose is folded into the operand loads (o is read in place). fp32
 * accumulation on the matrix cores, one rounding to out_dtype.
 * Supported: dtype ATTN_DTYPE_BF16, out_dtype bf16 or fp32, hd in {64, 128},
 * D a multiple of 64, operands under 2 GiB. Pointers 16-byte aligned.
 */
int attn_out_proj_fwd(const void* o, const void* w_o, void* y, int B, int T, int H, int hd, int D,
                      int dtype, int out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
