/*
 * fa.h -- C ABI of the MI355X (gfx950) tiled exact attention library (libteaf.so).
 *
 * Tiled exact attention computes O = softmax(Q K^T * scale + mask) V one query tile at a
 * time, streaming key/value tiles through on-chip memory and keeping a running maximum and
 * running sum per query row (online softmax), so the N x N score matrix never reaches HBM.
 * Sources: "ops-transformer" article (gitcode.csdn.net), section 二.1 "FlashAttention算子"
 * (conventional attention listing; tiled loop over Q blocks and K/V blocks with an online
 * softmax update and one final normalisation); zwxr.cn article on ops-transformer, section
 * 3.1 (running max m and normaliser l per row; fp16 scores with an fp32 softmax
 * denominator; prefetch of the next K/V block while the current one is computed).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers (HIP device memory) owned by the caller. The
 *    library allocates nothing and is thread-safe. Its mutable state is the HIP error code
 *    of the last failed launch, kept per calling thread (see fa_last_hip_error), and the
 *    per-GPU address of the static scratch array of fa_decode_paged_noalloc (looked up
 *    once per GPU, under a lock); raising a kernel's dynamic LDS limit (an idempotent
 *    runtime attribute) happens on every launch.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). All work is
 *    enqueued on it; calls return before the work completes.
 *  - Return value: FA_OK (0) or a negative fa_status. Argument checks run on the host BEFORE
 *    any launch; on error nothing is launched and no output is written. A launch failure is
 *    reported as FA_ERR_HIP. Faults inside a kernel surface at the caller's next
 *    synchronisation, as for any HIP work.
 *  - Contents of device buffers (page tables, sequence lengths) cannot be checked on the
 *    host. The paged entry points clamp page ids into the pool and lengths into their
 *    documented ranges, so a corrupt table gives wrong values but no access outside the
 *    buffers.
 */
#ifndef TEAF_FA_H
#define TEAF_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = -1,        /* a required pointer is NULL */
    FA_ERR_SHAPE = -2,       /* a size is out of range (B, H, N < 1, window < 1, ...) */
    FA_ERR_UNSUPPORTED = -3, /* valid but not built: head dim, dtype, mask, page size */
    FA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than the query function says */
    FA_ERR_HIP = -5,         /* the HIP runtime refused a launch */
    FA_ERR_SCRATCH = -6      /* fa_decode_paged_noalloc: more than its static scratch */
} fa_status;

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

/* Masks. Query row i of Nq sits at absolute position i' = i + (Nkv - Nq) (bottom-right
 * alignment, so a single decode query sees every key). Key j is visible when
 *   FA_MASK_NONE          : always;
 *   FA_MASK_CAUSAL        : j <= i'  (the diagonal is kept);
 *   FA_MASK_WINDOW_GLOBAL : j <= i' and (i' - j < window or j < n_global);
 *   FA_MASK_BAND          : i' - window <= j <= i' + window  (both sides of the query);
 *   FA_MASK_PREFIX_LM     : j <= i' or j < n_global  (n_global = prefix length).
 * The causal mask follows the LLaMA deployment in the ops-transformer article (section 四,
 * FlashAttention(causal=True): each token sees only earlier tokens and itself). The window
 * mask follows the sparse_config of the ascend-transformer-boost article (场景三:
 * sliding_window mode, window_size 2048, 64 global tokens such as BOS), read as a causal
 * window of `window` keys ending at the query plus the first `n_global` key positions. The
 * band mask is the band attention of the zwxr.cn article on ops-transformer (section 3.2:
 * each token attends the positions within +-w of it). Prefix LM is one of the sparse
 * variants the ascend-transformer-boost article names (场景三), read as: the first
 * n_global keys are visible to every query, later keys causally. */
typedef enum {
    FA_MASK_NONE = 0,
    FA_MASK_CAUSAL = 1,
    FA_MASK_WINDOW_GLOBAL = 2,
    FA_MASK_BAND = 3,
    FA_MASK_PREFIX_LM = 4
} fa_mask;

/*
 * fa_forward -- tiled exact attention forward pass.
 *
 *  q    [B, H, Nq,  d]  dtype, contiguous (row-major, d fastest)
 *  k    [B, H, Nkv, d]  dtype, contiguous
 *  v    [B, H, Nkv, d]  dtype, contiguous
 *  o    [B, H, Nq,  d]  dtype, written
 *  lse  [B, H, Nq]      float32, written: natural-log log-sum-exp of the scaled visible
 *                       scores of each row (-inf for a row with no visible key, whose O
 *                       row is then 0). Required (not NULL).
 *  scale       multiplies Q K^T (normally 1/sqrt(d)).
 *  mask_mode   fa_mask. FA_MASK_WINDOW_GLOBAL needs window >= 1 and n_global >= 0;
 *              FA_MASK_BAND needs window >= 0 (0: each row sees only its own position);
 *              FA_MASK_PREFIX_LM needs n_global >= 0 (0: causal). Unused ones are ignored.
 *  dtype       fa_dtype of q, k, v and o. Scores, softmax statistics and the output
 *              accumulator are float32 for every dtype; for fp16/bf16 the probabilities
 *              are rounded to the input dtype before the product with V.
 *  Supported: d in {64, 128}; any B, H, Nq, Nkv >= 1 (no padding needed; tails are
 *  masked inside the kernel); B*H*ceil(Nq/128) < 2^24 (workgroups of 256 threads, whose
 *  count a dispatch holds in 32 bits of work-items; the backward also needs
 *  B*H*ceil(Nkv/128) < 2^24, chunked prefill num_seqs*H*ceil(Qmax/128) < 2^24) and every
 *  tensor < 2^31 elements per (b, h); else FA_ERR_SHAPE.
 *  q, k, v, o need 16-byte alignment.
 */
int fa_forward(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
               int Nq, int Nkv, int d, float scale, int mask_mode, int window, int n_global,
               int dtype, void *stream);

/*
 * fa_forward_block_sparse -- block-sparse attention forward (one of the sparse variants the
 * ascend-transformer-boost article lists in 场景三; the pages name it without a format, read
 * here as a layout of visible tiles).
 *
 *  q, k, v, o, lse, B, H, Nq, Nkv, d, scale, dtype, stream: as fa_forward.
 *  layout  [H, ceil(Nq/block), ceil(Nkv/block)] uint8 DEVICE array, row-major: key j is
 *          visible from query row i of head h when layout[h][i/block][j/block] != 0. The
 *          same layout serves every batch entry. There is no shift between query and key
 *          positions (row i and key i share a block index). A row whose layout row is all
 *          zero gets O = 0 and LSE = -inf.
 *  block   tile edge in positions; only 128 is built (FA_ERR_UNSUPPORTED otherwise).
 *  Supported: as fa_forward, with Nkv <= 262144 (2048 key blocks; a workgroup keeps its
 *  list of visible key blocks on chip). The layout's contents are not checked on the host.
 */
int fa_forward_block_sparse(const void *q, const void *k, const void *v, void *o, float *lse,
                            int B, int H, int Nq, int Nkv, int d, float scale,
                            const uint8_t *layout, int block, int dtype, void *stream);

/*
 * fa_backward -- gradients dQ, dK, dV of fa_forward for the loss gradient dO.
 *
 * The pages keep the N x N scores out of memory and recompute them in the backward pass,
 * which they call cheap ("ops-transformer" article on gitcode.csdn.net, section 二.1: the
 * conventional scores would have to be read again in back-propagation; "ascend-transformer-
 * boost" article, 场景一: the checkpoint boundary sits on the FlashAttention output because
 * recomputing it costs little). Here P = exp(scale Q K^T - LSE) is rebuilt tile by tile from
 * the forward's LSE, and with D_i = sum_c dO_ic O_ic
 *   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dK = scale dS^T Q,  dQ = scale dS K.
 *
 *  q, k, v        as fa_forward (the same tensors the forward saw).
 *  o, lse         the forward's outputs for q, k, v with the same scale and mask.
 *  dout           [B, H, Nq, d] dtype: gradient of the loss with respect to o.
 *  dq             [B, H, Nq, d] dtype, written.
 *  dk, dv         [B, H, Nkv, d] dtype, written (zero for a key no query sees).
 *  B .. n_global  as fa_forward. A row with lse = -inf (no visible key) contributes nothing.
 *  dtype          FA_F16 or FA_BF16: products take fp16/bf16 operands (P and dS are
 *                 rounded to dtype) with float32 accumulation; the outputs are rounded
 *                 once at the end. FA_F32: float32 operands and products throughout (the
 *                 pages recommend fp32 or bf16 for training: ops-transformer article on
 *                 gitcode.csdn.net, section 三.2); a plain pair of kernels.
 *  workspace      device buffer of at least fa_backward_workspace_bytes(B, H, Nq) bytes
 *                 (per-row D and log2-scaled LSE, grouped by 32-row tile); contents need no
 *                 initialisation; 16-byte aligned.
 *  Supported: d in {64, 128}; masks FA_MASK_NONE .. FA_MASK_PREFIX_LM; sizes as fa_forward.
 *  Two kernels run on `stream`: dQ (which also forms the row statistics into the
 *  workspace), then dK/dV; no atomics, so the results are bitwise reproducible. All tensor
 *  pointers need 16-byte alignment.
 */
size_t fa_backward_workspace_bytes(int B, int H, int Nq);

int fa_backward(const void *q, const void *k, const void *v, const void *o, const float *lse,
                const void *dout, void *dq, void *dk, void *dv, int B, int H, int Nq, int Nkv,
                int d, float scale, int mask_mode, int window, int n_global, int dtype,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa_backward_block_sparse -- gradients of fa_forward_block_sparse: the recomputation of
 * fa_backward (same passages) with the visible keys of each query row given by the block
 * layout of fa_forward_block_sparse (the sparse variants of the "ascend-transformer-boost"
 * article, 场景三).
 *
 *  q .. dv, B, H, Nq, Nkv, d, scale, dtype, workspace, workspace_bytes, stream: as
 *          fa_backward; o and lse are fa_forward_block_sparse's outputs for the same layout.
 *  layout, block: as fa_forward_block_sparse (DEVICE array [H, ceil(Nq/block),
 *          ceil(Nkv/block)] uint8, one layout for every batch entry; block 128 only).
 *  Supported: as fa_backward, with Nq and Nkv <= 262144 (each workgroup lists the visible
 *  blocks of its row or column of the layout on chip). A key no query row sees gets dK = dV
 *  = 0, a row that sees no key dQ = 0. The layout's contents are not checked on the host.
 */
int fa_backward_block_sparse(const void *q, const void *k, const void *v, const void *o,
                             const float *lse, const void *dout, void *dq, void *dk, void *dv,
                             int B, int H, int Nq, int Nkv, int d, float scale,
                             const uint8_t *layout, int block, int dtype, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * fa_merge_lse -- combine two attention results over disjoint key sets of the same query
 * rows: lse = ln(e^lse_a + e^lse_b), o = e^(lse_a - lse) o_a + e^(lse_b - lse) o_b. This
 * is the step that lets the "ascend-transformer-boost" article (场景四) compute one
 * attention as separate calls over parts of the keys. A side with lse = -inf contributes
 * nothing; a row with -inf on both sides gets o = 0, lse = -inf.
 *
 *  o_a, o_b, o   [rows, d] dtype (o may alias o_a or o_b)
 *  lse_a, lse_b, lse  [rows] float32, natural log (lse may alias lse_a or lse_b)
 *  Supported: d in {64, 128}; dtype FA_F32, FA_F16, FA_BF16; rows >= 1 and
 *  rows * d * sizeof(dtype) / 16 <= 2^32 - 256 (one thread per 16 bytes of a row); o_a, o_b, o
 *  16-byte aligned. Arithmetic in float32; o is rounded to dtype once.
 */
int fa_merge_lse(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b,
                 void *o, float *lse, long long rows, int d, int dtype, void *stream);

/*
 * fa_multimodal_forward -- attention of image and text tokens with the multimodal pattern
 * of the "ascend-transformer-boost" article (场景四): image tokens attend to all image
 * tokens and no text; text tokens attend to all image tokens and causally to text tokens.
 * The article runs this as regular attention calls rather than one call with an irregular
 * mask; text_mode picks how the text part is computed:
 *  FA_MULTIMODAL_SPLIT_MERGE  the article's three calls, merged by log-sum-exp:
 *     1. image queries x image keys, no mask        -> o_img, lse_img
 *     2. text queries x text keys, causal           -> o_txt, lse_txt
 *     3. text queries x image keys, no mask         -> workspace
 *     4. fa_merge_lse of 2 and 3 into o_txt, lse_txt.
 *  FA_MULTIMODAL_FUSED  call 1, then calls 2 and 3 as ONE causal launch over n_img + n_txt
 *     keys whose key tiles come first from the image K/V and then from the text K/V (with
 *     bottom-right alignment every text row sees all image keys and the text keys up to
 *     itself): no merge, no workspace. Needs n_img % 32 == 0 and FA_F16 or FA_BF16
 *     (FA_ERR_UNSUPPORTED otherwise).
 * Both equal (up to rounding) one call over [image; text] with FA_MASK_PREFIX_LM and
 * n_global = n_img.
 *
 *  q_img, k_img, v_img  [B, H, n_img, d] dtype;  q_txt, k_txt, v_txt  [B, H, n_txt, d]
 *  o_img [B, H, n_img, d], lse_img [B, H, n_img]; o_txt [B, H, n_txt, d],
 *  lse_txt [B, H, n_txt]: written (lse float32).
 *  workspace  (split-merge only; may be NULL when fused) at least
 *             fa_multimodal_workspace_bytes(B, H, n_txt, d, dtype) bytes, 16-byte aligned,
 *             no initialisation needed (the text-to-image partial result).
 *  Supported: as fa_forward for each call (d in {64, 128}; FA_F32, FA_F16, FA_BF16).
 *  All argument checks run before the first launch; the kernels are enqueued in order on
 *  `stream`.
 */
typedef enum { FA_MULTIMODAL_SPLIT_MERGE = 0, FA_MULTIMODAL_FUSED = 1 } fa_multimodal_mode;

size_t fa_multimodal_workspace_bytes(int B, int H, int n_txt, int d, int dtype);

int fa_multimodal_forward(const void *q_img, const void *k_img, const void *v_img,
                          const void *q_txt, const void *k_txt, const void *v_txt, void *o_img,
                          float *lse_img, void *o_txt, float *lse_txt, int B, int H, int n_img,
                          int n_txt, int d, float scale, int dtype, int text_mode,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Paged single-token decode ("ascend-transformer-boost" article, 场景二: KV cache split
 * into fixed pages of 256 tokens, a new page per overflow, no reallocation; the attention
 * reads history K/V through the page layout). Each sequence has one query token at the
 * newest position, which sees all of its seq_lens[s] keys.
 *
 *  q           [S, H, d]                                  dtype
 *  k_pages     [num_pages, page_size, H, d]               dtype (physical page pool)
 *  v_pages     [num_pages, page_size, H, d]               dtype
 *  page_table  [S, max_pages_per_seq] int32, row-major: logical page p of sequence s is
 *              physical page page_table[s*max_pages_per_seq + p]; only the first
 *              ceil(seq_lens[s]/page_size) entries of a row are read.
 *  seq_lens    [S] int32, each in [1, max_pages_per_seq*page_size]
 *  o           [S, H, d]                                  dtype, written
 *  lse         [S, H] float32, written; may be NULL.
 *  workspace   device buffer of at least fa_decode_paged_workspace_bytes(...) bytes for
 *              the per-split partial results (split-KV); contents need no initialisation.
 *  Supported: page_size == 256, d == 128, dtype FA_F16 or FA_BF16, H a multiple of 8;
 *  S, H and max_pages_per_seq at most 65535 each (so up to 16,776,960 tokens a sequence:
 *  these are launch-grid dimensions), else FA_ERR_SHAPE.
 *  The kernels never read page slots at or past seq_lens[s], nor unused table entries.
 *  Page ids outside [0, num_pages) are clamped into the pool (wrong values, never a read
 *  outside it); a length past max_pages_per_seq*page_size counts as that maximum, and a
 *  length below 1 gives o = 0 and lse = -inf for that sequence.
 *  Two kernels run on `stream`: the split pass writes partial (O, LSE) per split of
 *  the keys; the combine pass merges them by log-sum-exp and writes o and lse.
 */
size_t fa_decode_paged_workspace_bytes(int num_seqs, int H, int d, int max_pages_per_seq,
                                       int page_size);

int fa_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                    const int32_t *page_table, const int32_t *seq_lens, void *o, float *lse,
                    int page_size, int num_seqs, int H, int d, int max_pages_per_seq,
                    int num_pages, float scale, int dtype, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * fa_decode_paged_noalloc -- fa_decode_paged without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). It calls no allocating routine: the split partials go to a
 * file-scope static device array of 16 MiB inside the library, one per GPU, held until the
 * process ends (its address is looked up once per GPU, on the first call there).
 *
 *  Arguments as fa_decode_paged, without workspace and workspace_bytes; same kernels,
 *  same results bit for bit.
 *  Limit: the partials take num_seqs * H * ceil(max_pages_per_seq * 256 / split) * (d + 1)
 *  * 4 bytes, split being the token run per workgroup the launch picks (256, 128 or 64:
 *  the longest that still gives at least 512 workgroups). Every call with
 *  num_seqs * H * max_pages_per_seq <= 8128 fits; larger ones fit when the longer splits
 *  are picked (up to 32512 at split 256). A call that does not fit returns FA_ERR_SCRATCH
 *  before anything is launched.
 *  Concurrency: every call on one GPU uses that GPU's one array, so calls that can overlap
 *  on a GPU (other streams, other threads) race and must be serialised by the caller.
 *  Nothing in the array needs clearing between calls.
 */
int fa_decode_paged_noalloc(const void *q, const void *k_pages, const void *v_pages,
                            const int32_t *page_table, const int32_t *seq_lens, void *o,
                            float *lse, int page_size, int num_seqs, int H, int d,
                            int max_pages_per_seq, int num_pages, float scale, int dtype,
                            void *stream);

/*
 * fa_prefill_paged -- multi-token (chunked) prefill against the paged KV cache of
 * fa_decode_paged. The pages' inference loop (ascend-transformer-boost article, 场景二) feeds
 * tokens into a layer whose KV cache is paged; a chunk of several new tokens per sequence is
 * the multi-token form of that step. The chunk's K/V rows must already be in the cache: the
 * chunk is the newest q_lens[s] of the seq_lens[s] cached tokens, so query row i of sequence
 * s sits at absolute position i + seq_lens[s] - q_lens[s] and the masks of fa_mask apply
 * with that bottom-right alignment (FA_MASK_CAUSAL: the chunk sees the whole history and
 * itself causally).
 *
 *  q           [S, Qmax, H, d]  dtype: row i < q_lens[s] of sequence s is a query token
 *  k_pages,
 *  v_pages     [num_pages, page_size, H, d]  dtype (as fa_decode_paged)
 *  page_table  [S, max_pages_per_seq] int32 (as fa_decode_paged)
 *  seq_lens    [S] int32, each in [1, max_pages_per_seq * page_size]
 *  q_lens      [S] int32, each in [0, min(Qmax, seq_lens[s])]
 *  o           [S, Qmax, H, d]  dtype, written for rows i < q_lens[s] (others untouched)
 *  lse         [S, Qmax, H] float32, written for the same rows (-inf: no visible key)
 *  scale, mask_mode, window, n_global, dtype: as fa_forward (masks NONE .. PREFIX_LM).
 *  Supported: page_size == 256; d in {64, 128}; dtype FA_F16 or FA_BF16; H <= 65535;
 *  q, k_pages, v_pages and o 16-byte aligned. One kernel runs on `stream`; it reads no
 *  page slot at or past seq_lens[s] and no table entry past ceil(seq_lens[s]/page_size).
 *  Page ids outside [0, num_pages) are clamped into the pool (wrong values, never a read
 *  outside it); the lengths are clamped to the ranges above.
 */
int fa_prefill_paged(const void *q, const void *k_pages, const void *v_pages,
                     const int32_t *page_table, const int32_t *seq_lens, const int32_t *q_lens,
                     void *o, float *lse, int page_size, int num_seqs, int Qmax, int H, int d,
                     int max_pages_per_seq, int num_pages, float scale, int mask_mode,
                     int window, int n_global, int dtype, void *stream);

/* Static text for a status code (never NULL). */
const char *fa_status_string(int status);

/* Text of the HIP error behind the calling thread's most recent FA_ERR_HIP ("no error" if
 * none). The pointer is static; the text stays valid until the thread's next failing call. */
const char *fa_last_hip_error(void);

/* Library ABI version: major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TEAF_FA_H */
