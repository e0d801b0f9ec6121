/*
 * libfattn -- exact attention for AMD MI355X (gfx950), C ABI.
 *
 * Every entry point is asynchronous on the HIP stream it is given
 * (hipStream_t passed as void*; NULL means the default stream).  All tensor
 * pointers are DEVICE pointers owned by the caller; the library never
 * allocates, frees or retains device memory and keeps no state between calls
 * apart from a thread-local error string.  Calls are re-entrant and may run
 * on concurrent streams.
 *
 * Arguments are validated on the host before anything is launched; an
 * invalid call launches nothing and returns a non-zero status.  Values that
 * live in device memory (sequence lengths, block tables, offsets) are not
 * read by the host: kernels clamp them to the sizes passed in (for the jagged
 * layout, to the total offsets[B]; see attn_hstu_jagged), so a violated
 * precondition gives unspecified output but no access outside the sizes the
 * call describes.  Kernel faults surface at the caller's next
 * synchronisation.
 *
 * Element types: "bf16" is IEEE-style bfloat16 stored as uint16; "f32" is
 * IEEE binary32.  Every tensor is dense and contiguous in the layout given,
 * and every tensor pointer must be 16-byte aligned.
 */
#ifndef FATTN_H
#define FATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define FATTN_OK 0
#define FATTN_ERR_INVALID_ARG 1 /* argument out of its documented range        */
#define FATTN_ERR_UNSUPPORTED 2 /* valid, but no kernel for it (e.g. d = 96)   */
#define FATTN_ERR_HIP 3         /* HIP reported an error at launch             */
#define FATTN_ERR_INTERNAL 4

/*
 * attn_fwd -- fused exact attention, bf16 in / bf16 out, fp32 accumulation.
 *
 *   O = softmax(scale * Q K^T [+ causal mask]) V,   LSE = m + ln(sum exp(s - m))
 *
 * The operation is the standard attention formula (FlashAttention (TH) page,
 * the section on standard attention; ledger page, "FLOPs" section), computed
 * as one tiled kernel with an online softmax (CANN ops-transformer
 * FlashAttention page, steps 1-4 of the solution) so that the N x N score
 * matrix never reaches device memory.  The causal mask is generated in the
 * kernel and tiles above the diagonal are skipped (HSTU page, optimisation
 * two, in-kernel mask).
 *
 *   q    bf16 [B, H,   N, d]
 *   k, v bf16 [B, Hkv, N, d]   query head h reads key/value head h / (H/Hkv)
 *   o    bf16 [B, H,   N, d]   written
 *   lse  f32  [B, H,   N]      written (natural log), or NULL to skip
 *   H % Hkv == 0; d in {64, 128, 256}; scale finite and >= 0;
 *   causal in {0, 1}: 1 lets row i see keys j <= i.
 *   B == 0 or N == 0 is a valid empty call (nothing launched).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Hkv, int N, int d, float scale, int causal,
             void* stream);

/*
 * attn_fwd_f32 -- the same operation with f32 q, k, v, o (same layouts), f32
 * arithmetic throughout (probabilities are not rounded).  d == 64 only.
 */
int attn_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Hkv, int N, int d, float scale, int causal,
                 void* stream);

/*
 * attn_fwd_fp8 -- attn_fwd with FP8 inputs: q, k, v in OCP FP8 E4M3 (one
 * byte each), one f32 descale per (batch, head) slice of each (the real value
 * is fp8 * descale), both products on the FP8 matrix cores with f32
 * accumulation, o in bf16.  The FlashAttention (TH) page's FlashAttention-3
 * section names FP8 as a lever but gives no scaling convention; this is the
 * per-head one.  The probabilities are rounded to E4M3 before the P V
 * product, which bounds the accuracy (about 2^-4 relative per weight).
 *
 *   q          E4M3 [B, H, N, d];  descale_q f32 [B, H]   (device memory)
 *   k, v       E4M3 [B, Hkv, N, d]; descale_k, descale_v f32 [B, Hkv]
 *   o          bf16 [B, H, N, d] written;  lse f32 [B, H, N] written, or NULL
 *   d == 128; the other arguments as attn_fwd.  Descales are read on the
 *   device; they must be finite and > 0.
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                 const float* descale_q, const float* descale_k, const float* descale_v,
                 int B, int H, int Hkv, int N, int d, float scale, int causal,
                 void* stream);

/*
 * attn_decode_workspace_bytes -- device workspace attn_decode and
 * attn_decode_paged need: room for one partial output row (f32, d values) and
 * one partial log-sum-exp (f32) per (head, slot), B * (num_splits + 1) slots
 * per head, rounded up to 256 bytes.  num_splits == 0 asks for room for the
 * automatic choice of either entry point, which is at most 64 splits.
 * Returns 0 for an invalid shape (B < 0, H < 1, d < 1, num_splits outside
 * 0..64).
 */
size_t attn_decode_workspace_bytes(int B, int H, int d, int num_splits);

/*
 * attn_decode -- one new query token per sequence against a KV cache,
 * split over the key length, then merged by log-sum-exp weights.
 *
 * Decode is the bandwidth-bound step the ledger page describes (bandwidth
 * section: s_j = q^T k_j over all history keys, o = sum_j p_j v_j, O(n d)
 * bytes per step), and prefill and decode take different kernels (CANN
 * ops-transformer FlashAttention page, prefill vs decode).  Kernel 1 lays the
 * 32-key blocks of all sequences end to end and gives each (kv-head, work
 * item) an equal run of them, B * num_splits items per kv head, so the work is
 * even whatever the lengths; for each sequence its run touches it writes a
 * normalised partial output and its log-sum-exp to the workspace; kernel 2
 * combines the partials of each (sequence, head).
 *
 *   q          bf16 [B, H, d]            (one token per sequence)
 *   k_cache    bf16 [B, Hkv, Lmax, d]
 *   v_cache    bf16 [B, Hkv, Lmax, d]
 *   seqlens_k  int32 [B], device memory; the query attends to cache rows
 *              [0, seqlens_k[b]); rows at or beyond it are never read.
 *              Values are clamped to [0, Lmax]; a sequence of length 0 gives
 *              O = 0 and LSE = -inf.
 *   o          bf16 [B, H, d]            written
 *   lse        f32  [B, H]               written, or NULL
 *   H % Hkv == 0 with H/Hkv in {1, 2, 4, 8, 16, 32} (32: multi-query
 *              attention with 32 heads); d == 128; scale finite, >= 0.
 *   num_splits 0 = automatic, else 1..64: the average number of chunks
 *              (work items) per sequence.  The T 32-key blocks of the batch
 *              (ceil(seqlens_k[b] / 32) per sequence, summed) are cut into
 *              min(B * num_splits, T) equal runs of floor/ceil(T / items)
 *              blocks, so sequences of equal length get num_splits chunks
 *              each and longer sequences more.  Automatic: about 768 work
 *              items in all (1024 for the paged cache), i.e. 768 / (B * Hkv)
 *              chunks per sequence, at most 64 -- measured faster than a
 *              fixed 16 on the GQA decode workload -- raised for very long
 *              caches.  A count whose work items would span 2^32 bytes of one
 *              kv head returns FATTN_ERR_UNSUPPORTED.
 *   workspace  device buffer of at least
 *              attn_decode_workspace_bytes(B, H, d, num_splits) bytes;
 *              contents on entry are ignored.
 */
int attn_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* seqlens_k, void* o, float* lse,
                int B, int H, int Hkv, int Lmax, int d, float scale,
                int num_splits, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * attn_decode_noalloc -- attn_decode without a caller-supplied workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The partials live
 * in a static device array of 32 MiB per GPU that the library owns and keeps
 * until the process ends; the call itself allocates nothing.
 *
 *   Arguments as attn_decode, without workspace and workspace_bytes.
 *   A call whose workspace, attn_decode_workspace_bytes(B, H, d, splits) for
 *   the split count it uses, exceeds 32 MiB returns FATTN_ERR_UNSUPPORTED
 *   (use fewer splits, or attn_decode).  The first call on each device looks
 *   up the array's device address (hipGetSymbolAddress) with that device
 *   current.  All calls on one device share the array: calls that may overlap
 *   on one device (several streams, several host threads) race and must be
 *   ordered by the caller.
 */
int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seqlens_k, void* o, float* lse,
                        int B, int H, int Hkv, int Lmax, int d, float scale,
                        int num_splits, void* stream);

/*
 * attn_decode_paged -- attn_decode over a paged KV cache.
 *
 * The cache lives in fixed-size pages found through a per-sequence block
 * table (the PagedAttention scheme that the CANN ops-transformer FlashAttention
 * page lists under KV-cache management, Kwon et al. 2023 in the FlashAttention
 * (TH) page's bibliography).  The result is that of attn_decode on the cache
 * gathered in logical order; the split kernel reads each page in place.
 *
 *   k_pages, v_pages  bf16 [num_pages, Hkv, page_size, d]
 *   block_table       int32 [B, max_pages_per_seq], device memory: logical
 *                     page p of sequence b (keys p*page_size .. +page_size-1)
 *                     is physical page block_table[b][p]; entries are clamped
 *                     to [0, num_pages).
 *   seqlens_k         int32 [B], device memory, clamped to
 *                     [0, max_pages_per_seq * page_size]; keys at or beyond
 *                     it are never read, even inside the last page.
 *   page_size         a power of two in [16, 1024].
 *   q, o, lse, H, Hkv, d, scale, num_splits: as attn_decode, with
 *   Lmax = max_pages_per_seq * page_size.  Workspace: at least
 *   attn_decode_workspace_bytes(B, H, d, num_splits) bytes.
 *   A split may span at most 2047 pages; a call whose splits would span more
 *   returns FATTN_ERR_UNSUPPORTED (use more splits or larger pages).
 */
int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                      const int32_t* block_table, const int32_t* seqlens_k,
                      void* o, float* lse, int B, int H, int Hkv, int page_size,
                      int max_pages_per_seq, int num_pages, int d, float scale,
                      int num_splits, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * attn_hstu_jagged -- HSTU pointwise attention over packed variable-length
 * sequences (no padding).
 *
 * Per sequence b and head h, following the order of the HSTU page's listing
 * (x = Q K^T; x *= alpha; x = silu(x); x *= mask / n; O = x V) with the mask
 * generated in the kernel (optimisation two) and the sequences packed by
 * offsets (optimisation three, jagged tensors):
 *
 *   O[t] = inv_n * sum_{j visible from t} silu(alpha * q_t . k_j) v_j
 *
 * with silu(x) = x / (1 + e^-x); there is no softmax and no LSE.  The kernel
 * multiplies q by alpha * log2(e) once and rounds it to bf16 before the
 * product (a relative change of at most 2^-9 per element), and rounds each
 * weight to bf16 before the product with V.
 *
 *   q, k, v   bf16 [T, H, d] packed: sequence b owns rows
 *             [offsets[b], offsets[b+1])
 *   o         bf16 [T, H, d]  written (rows of every sequence)
 *   offsets   int32 [B + 1], device memory, non-decreasing, offsets[0] = 0,
 *             offsets[B] = T.  The kernels read offsets[B] as the row count
 *             and clamp every offsets[b] into [0, offsets[B]] and every
 *             length to >= 0, so no row outside [0, offsets[B]) is touched;
 *             offsets[B] itself must not exceed the rows of q, k, v and o
 *             (the library cannot check it).
 *   max_seqlen >= every sequence length (rows beyond it are not computed)
 *   d in {64, 128}; alpha, inv_n finite; causal in {0, 1} (1: key j <= row i).
 */
int attn_hstu_jagged(const void* q, const void* k, const void* v, void* o,
                     const int32_t* offsets, int B, int H, int d, int max_seqlen,
                     float alpha, float inv_n, int causal, void* stream);

/*
 * attn_bwd_workspace_bytes -- device workspace attn_bwd needs: two f32 arrays
 * over the B*H*N query rows, each rounded up to 256 bytes (the row sums
 * delta below, and each row's -LSE log2(e), which the key-block kernel reads
 * instead of scaling the LSE itself).  Returns 0 for an invalid shape.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int N);

/*
 * attn_bwd -- gradients of attn_fwd with respect to q, k and v.
 *
 * The pages name the backward pass only by its cost (ledger page, memory
 * section: training keeps n x n backward intermediates besides S and P);
 * this entry point computes it without them.  With P = exp(scale Q K^T -
 * LSE) recomputed from the forward's LSE (masked as in the forward):
 *
 *   dV = P^T dO,  dP = dO V^T,  delta_i = sum_c dO_ic O_ic,
 *   dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q,
 *
 * and for grouped-query attention a key/value head's gradients sum over
 * the query heads that read it.
 *
 *   q, o, dout   bf16 [B, H,   N, d]  (o and lse as written by attn_fwd
 *                                      with the same arguments)
 *   k, v         bf16 [B, Hkv, N, d]
 *   lse          f32  [B, H,   N]     natural log, as from attn_fwd
 *   dq           bf16 [B, H,   N, d]  written
 *   dk, dv       bf16 [B, Hkv, N, d]  written
 *   workspace    device buffer of at least attn_bwd_workspace_bytes(B, H, N)
 *                bytes; contents on entry are ignored (it receives delta and
 *                -LSE log2(e) per row).
 *   H % Hkv == 0; d in {64, 128}; scale finite and >= 0; causal in {0, 1}.
 *   B == 0 or N == 0 is a valid empty call.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dout, void* dq, void* dk, void* dv,
             int B, int H, int Hkv, int N, int d, float scale, int causal,
             void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* fattn_status_string(int status);

/* Message describing the last failed call on this thread ("" if none). */
const char* fattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FATTN_H */
