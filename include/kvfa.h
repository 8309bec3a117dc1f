/*
 * kvfa.h — C ABI of the exact-attention library (libkvfa.so) for AMD MI355X (gfx950).
 *
 * The library computes exact attention, O = softmax(scale * Q K^T) V with row-wise
 * softmax, as defined on the page "Donanıma Duyarlı Algoritma Tasarımı:
 * FlashAttention" (section "Transformer Mimarisi ve Self-Attention Mekanizması"),
 * the FlashAttention way: Q, K and V are processed in tiles held on chip and a
 * running row maximum and row sum ("Online Softmax Prensibi", steps 1-5) replace the
 * materialised score matrix. Besides O it returns the per-row softmax statistics
 * that page keeps in HBM (section "FlashAttention-1 (İki Geçişli Yaklaşım)") as one
 * natural-log log-sum-exp per row: lse = M + ln L.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named as tensors are DEVICE pointers, allocated and owned by the caller.
 *   The library never allocates or frees device memory and keeps no global mutable
 *   state; calls on different streams are independent.
 * - Every tensor is dense and row-major with the head dimension d innermost; there
 *   are no stride arguments. bf16 tensors are passed as raw 16-bit patterns.
 * - Tensor pointers must be 16-byte aligned. lse may be NULL (then it is not written).
 * - stream is the HIP stream the work is enqueued on (NULL = the default stream) and
 *   must belong to the current device, as for any HIP call. Work is only enqueued: a
 *   return of FA_OK means "launched", device-side results are ready after the
 *   caller synchronises the stream.
 * - Errors: invalid arguments return FA_ERR_INVALID or FA_ERR_UNSUPPORTED before
 *   anything is enqueued (no output is touched); a failed launch returns
 *   FA_ERR_HIP. Nothing crosses the ABI as an exception.
 * - Causal masking is bottom-right aligned: query i sits at absolute position
 *   Nk - Nq + i and attends keys j <= i + (Nk - Nq) (new queries come after the
 *   cached keys, as in the KV-cache flow of the glossary entry "KV Cache
 *   (Anahtar-Değer Önbelleği)", yapayzekasozluk.tr/etiket/attention).
 * - Grouped-query attention (same glossary entry: several query heads share one
 *   K-V head): query head h reads K/V head h / (H / Hkv); H % Hkv must be 0.
 */
#ifndef KVFA_H
#define KVFA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID = -1,      /* an argument is out of its documented range           */
    FA_ERR_UNSUPPORTED = -2,  /* a valid request the library does not implement      */
    FA_ERR_HIP = -3,          /* the HIP runtime reported an error at launch          */
    FA_ERR_SCRATCH = -4       /* fa_decode_paged_noalloc: request exceeds its scratch */
} fa_status;

/*
 * fa_fwd — bf16 prefill attention, fp32 accumulation.
 *   q   [B, H,   Nq, d] bf16        o   [B, H, Nq, d] bf16 (written)
 *   k   [B, Hkv, Nk, d] bf16        lse [B, H, Nq]    fp32 (written; may be NULL)
 *   v   [B, Hkv, Nk, d] bf16
 * d must be 64 or 128 (else FA_ERR_UNSUPPORTED). B, H, Hkv, Nq, Nk >= 1;
 * causal requires Nq <= Nk; scale must be finite and > 0 (normally 1/sqrt(d));
 * Nk * d * 2 and Nq * d * 2 must each be below 2^31 bytes (one head's slice).
 * Scores, the softmax and the accumulator are fp32; P and O are rounded to bf16
 * with round-to-nearest-even.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
           hipStream_t stream);

/*
 * fa_bwd — gradients of fa_fwd's output with respect to q, k and v, recomputing the
 * attention probabilities from q, k and the forward's lse instead of storing them (page
 * "Donanıma Duyarlı Algoritma Tasarımı: FlashAttention": only the per-row statistics of
 * the forward stay in HBM; glossary entry "Flash Attention": intermediates are
 * recomputed in the backward pass rather than saved). With P = exp(scale q k^T - lse)
 * (masked entries 0) and D = rowsum(dO * O):
 *   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,
 * dK and dV summed over the query heads of each GQA group.
 *   q, o, dout, dq  [B, H, Nq, d] bf16      k, v, dk, dv  [B, Hkv, Nk, d] bf16
 *   lse             [B, H, Nq] fp32, the forward's (natural-log) lse for these q, k, v
 *   workspace       device scratch of at least fa_bwd_workspace_size(B, H, Nq) bytes
 * Same ranges and errors as fa_fwd; lse, dout, dq, dk, dv and workspace must be non-NULL
 * and aligned (16 bytes; workspace 4), else FA_ERR_INVALID. dq, dk, dv are written (not
 * accumulated into); gradients are accumulated in fp32 and rounded to bf16. Three
 * kernels on the stream: D, then dK/dV, then dQ; deterministic (no atomics).
 */
size_t fa_bwd_workspace_size(int B, int H, int Nq);

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq,
           int Nk, int d, int causal, float scale, void* workspace, size_t workspace_bytes,
           hipStream_t stream);

/*
 * fa_fwd_two_pass — fa_fwd computed in the two passes of FlashAttention-1 (page
 * "Donanıma Duyarlı Algoritma Tasarımı: FlashAttention", section "FlashAttention-1
 * (İki Geçişli Yaklaşım)"): the first pass reads Q and K and writes only each row's
 * softmax statistics to HBM; the second reads Q, K, V and those statistics again,
 * recomputes the scores, normalises them with the statistics and accumulates the
 * output. It costs one more Q.K^T than fa_fwd and serves as an independent check of the
 * single-pass recurrence.
 * Same layouts, ranges and errors as fa_fwd, except that lse is REQUIRED (NULL gives
 * FA_ERR_INVALID): the statistics travel between the passes through it, as
 * lse = M + ln L, and it holds the result's lse on return. Numerics: as fa_fwd, with P
 * normalised before its rounding to bf16.
 */
int fa_fwd_two_pass(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                    hipStream_t stream);

/*
 * fa_fwd_window — fa_fwd with a sliding-window mask (glossary entry "Kayan Pencere
 * Dikkati (Sliding Window Attention)", yapayzekasozluk.tr/etiket/attention: each token
 * attends only the tokens within a fixed distance of its own position, so the work is
 * O(N w) instead of O(N^2)). Query i sits at position p = Nk - Nq + i (bottom-right, as
 * for causal) and attends keys j with p - window_left <= j <= p + window_right; -1 makes
 * a side unbounded. The symmetric window of width w is (w/2, w/2); a causal sliding
 * window is (w_left, 0); (-1, 0) is plain causal and (-1, -1) no mask at all.
 * Same layouts, numerics and errors as fa_fwd; additionally Nq <= Nk and
 * window_left, window_right >= -1 (else FA_ERR_INVALID). Every query attends at least
 * its own position, so no row is empty.
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Hkv, int Nq, int Nk, int d, int window_left,
                  int window_right, float scale, hipStream_t stream);

/*
 * fa_fwd_fp32 — the same operation with fp32 inputs and outputs and fp32 arithmetic
 * throughout (no reduced-precision step). Same layouts, ranges and errors as fa_fwd.
 */
int fa_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse,
                int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                hipStream_t stream);

/*
 * fa_decode_paged — one new query token per sequence against a paged KV cache
 * (glossary entry "KV Cache (Anahtar-Değer Önbelleği)": token n+1 reads the cached
 * K/V of the tokens before it; the cache is kept in fixed-size pages).
 *   q          [num_seqs, H, d] bf16
 *   k_cache    [num_pages, page_size, Hkv, d] bf16; token t of sequence s is slot
 *   v_cache     t % page_size of physical page page_table[s][t / page_size]
 *   page_table [num_seqs, max_pages_per_seq] int32
 *   seq_lens   [num_seqs] int32, device memory: cached tokens per sequence, the
 *              current token's K/V already appended (the query attends all of them)
 *   o          [num_seqs, H, d] bf16 (written)   lse [num_seqs, H] fp32 (may be NULL)
 *   workspace  device scratch of at least fa_decode_paged_workspace_size(...) bytes,
 *              owned by the caller; its contents on entry do not matter.
 * Work is split over the KV length (split-K: every work-group reads an equal range of
 * the cached pages, read from seq_lens on the device); the partial results are merged by
 * their log-sum-exps in a second kernel on the same stream (for more than 64 sequences a
 * small planning kernel runs first). Nothing is allocated and nothing synchronises.
 * Numerics: scores, the softmax, the accumulators and the merge are fp32; P is rounded to
 * bf16 (round-to-nearest-even) for the P.V products, O to bf16 at the end.
 * Requirements: page_size == 16 and d in {64, 128} (else FA_ERR_UNSUPPORTED);
 * H % Hkv == 0 and H / Hkv <= 16, or a multiple of 16; num_seqs, H, Hkv,
 * num_pages >= 1; max_pages_per_seq * page_size >= max_seq_len >= 1;
 * num_seqs <= 65535 and num_seqs * ceil(max_seq_len / 16) <= 248 * 65535 (the pages the
 * table can describe must fit the launch; else FA_ERR_UNSUPPORTED).
 * Device-side values: a seq_len outside [0, max_seq_len] is clamped into it; a
 * sequence with seq_len 0 gets O = 0 and lse = -inf; page ids outside
 * [0, num_pages) are never dereferenced (their tokens are skipped, so the result is
 * then not meaningful). Table entries past a sequence's last page and page slots
 * past its length are never read.
 */
size_t fa_decode_paged_workspace_size(int num_seqs, int H, int d, int max_seq_len,
                                      int page_size);

int fa_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* page_table, const int32_t* seq_lens, int page_size,
                    void* o, float* lse, int num_seqs, int H, int Hkv, int d,
                    int num_pages, int max_pages_per_seq, int max_seq_len, float scale,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_decode_paged_fp8 — fa_decode_paged on a cache stored in 8-bit floating point
 * (glossary entry "KV Cache (Anahtar-Değer Önbelleği)": quantising the KV cache to
 * INT8/FP8 cuts its memory 2-4x). Each cached element is one byte in the OCP e4m3 format
 * (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, 0x7f/0xff
 * NaN); its value is the decoded byte times the scale of its KV head:
 *   k_cache, v_cache  [num_pages, page_size, Hkv, d] uint8 (e4m3)
 *   k_scale, v_scale  [Hkv] fp32, device memory; finite and >= 0
 * Everything else (q, o, lse, page_table, seq_lens, workspace and its size, errors,
 * device-side behaviour) is as for fa_decode_paged. The result is the attention of the
 * dequantised cache: bytes are converted exactly, the numerics are those of
 * fa_decode_paged, the K scale is folded into the softmax scale and the V scale into each
 * partial result.
 * k_scale or v_scale NULL or misaligned: FA_ERR_INVALID.
 */
int fa_decode_paged_fp8(const void* q, const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale,
                        const int32_t* page_table, const int32_t* seq_lens, int page_size,
                        void* o, float* lse, int num_seqs, int H, int Hkv, int d,
                        int num_pages, int max_pages_per_seq, int max_seq_len, float scale,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_decode_paged_noalloc — fa_decode_paged for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It takes no workspace argument: the decode workspace lives in a static
 * device array of FA_NOALLOC_SCRATCH_BYTES, one per GPU the library runs on, held until
 * the process ends. The call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its first call on a device looks up that device's array
 * address once.
 * Arguments, layouts, numerics, device-side behaviour and errors are those of
 * fa_decode_paged (same kernels, same results bit for bit), except that a call whose
 * workspace, fa_decode_paged_workspace_size(num_seqs, H, d, max_seq_len, page_size),
 * would exceed FA_NOALLOC_SCRATCH_BYTES returns FA_ERR_SCRATCH before anything is
 * enqueued (the 64-sequence, H32, d 128, 8192-token decode needs about 35 MB).
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams or from different threads) race and must be serialised by the
 * caller. Calls in order on one stream are safe.
 */
#define FA_NOALLOC_SCRATCH_BYTES (64u << 20)

int fa_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* page_table, const int32_t* seq_lens, int page_size,
                            void* o, float* lse, int num_seqs, int H, int Hkv, int d,
                            int num_pages, int max_pages_per_seq, int max_seq_len, float scale,
                            hipStream_t stream);

/* The fewest cached tokens one split-K work-group's range holds for these sizes (a
 * multiple of the page size: 4 pages, or 1/32 of max_seq_len's pages, at most 248 pages).
 * The cached pages of all sequences, end to end, are cut into equal ranges of at least
 * this many tokens, one per work-group; a sequence is thereby cut into at most
 * ceil(max_seq_len / split) + 1 pieces, and the workspace holds that many partial results
 * per head, plus one int32 per sequence (its slot count) and a plan of 4 + 2 x max(1536,
 * ceil(num_seqs x max_pages / 248), num_seqs) int32 (for more than 64 sequences a small
 * planning kernel writes where each work-group's range starts). */
int fa_decode_paged_split_tokens(int num_seqs, int max_seq_len, int page_size);

/*
 * fa_fwd_paged — chunked prefill: bf16 attention of Nq new queries per sequence against
 * all of that sequence's cached keys, read through the page table (the prompt is fed
 * in chunks, each chunk's K/V first appended with fa_kv_append; glossary entry "KV
 * Cache (Anahtar-Değer Önbelleği)": later tokens read the stored K/V of earlier ones).
 *   q          [B, H, Nq, d] bf16          o [B, H, Nq, d] bf16 (written)
 *   k_cache,   [num_pages, page_size, Hkv, d] bf16, the layout of fa_decode_paged
 *   v_cache
 *   page_table [B, max_pages_per_seq] int32
 *   seq_lens   [B] int32, device memory: cached tokens of each sequence INCLUDING the
 *              Nq new ones, which are its last Nq tokens (query i sits at position
 *              seq_len - Nq + i; causal masking is bottom-right as everywhere)
 *   lse        [B, H, Nq] fp32 (written; may be NULL)
 * Numerics as fa_fwd. Requirements: page_size == 16, d in {64, 128} (else
 * FA_ERR_UNSUPPORTED); B, H, Hkv, Nq, num_pages >= 1; H % Hkv == 0;
 * Nq <= max_seq_len <= max_pages_per_seq * page_size; Nq * d * 2 < 2^31.
 * Device-side values: a seq_len outside [Nq, max_seq_len] is clamped into it; pages
 * with ids outside [0, num_pages) load as zeros (the result is then not meaningful);
 * table entries past a sequence's last page and slots past its length are never read.
 */
int fa_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* page_table, const int32_t* seq_lens, int page_size, void* o,
                 float* lse, int B, int H, int Hkv, int Nq, int d, int num_pages,
                 int max_pages_per_seq, int max_seq_len, int causal, float scale,
                 hipStream_t stream);

/*
 * fa_kv_append — store the keys and values of n_new new tokens per sequence in the
 * paged cache (glossary entry "KV Cache (Anahtar-Değer Önbelleği)": each token's K/V
 * is computed once and kept for every later step). A bit-exact copy, no arithmetic.
 *   k_new, v_new [num_seqs, n_new, Hkv, d] bf16 (read)
 *   k_cache,     [num_pages, page_size, Hkv, d] bf16 (the new slots are written)
 *   v_cache
 *   page_table   [num_seqs, max_pages_per_seq] int32; the pages that will hold the new
 *                tokens must already be assigned by the caller
 *   start_pos    [num_seqs] int32, device memory: position of the first new token of
 *                each sequence (its cached length before the call)
 * Token t of sequence s goes to slot (start_pos[s] + t) % page_size of page
 * page_table[s][(start_pos[s] + t) / page_size].
 * Requirements: page_size == 16, d in {64, 128} (else FA_ERR_UNSUPPORTED);
 * num_seqs, n_new, Hkv, num_pages, max_pages_per_seq >= 1.
 * Device-side values: a token whose position is negative or past the table
 * (>= max_pages_per_seq * page_size), or whose page id is outside [0, num_pages), is
 * not written. Two tokens mapped to the same slot (a table that shares a page being
 * written) race; which one lands is unspecified.
 */
int fa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                 const int32_t* page_table, const int32_t* start_pos, int page_size,
                 int num_seqs, int n_new, int Hkv, int d, int num_pages,
                 int max_pages_per_seq, hipStream_t stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVFA_H */
