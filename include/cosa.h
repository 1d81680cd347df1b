/*
 * cosa.h - C ABI of a gfx950 (MI355X) library for CoSA block-sparse causal
 * prefill attention over a paged KV cache.
 *
 * The method is described in "CoSA: Accelerating Long-Context Inference via
 * Proxy-Kernel Co-Designed Sparse Attention" (paper text on paperpeel.com):
 *   - the Kernel-Aware Proxy (KAP, §4.2 and App. C.1) scores key blocks for
 *     every query block and emits a computation-order mask M_KAP, with the
 *     "have rowmax" (HRM) blocks first, truncated to a stage-1 budget;
 *   - the Ordered-Skipping Kernel (OSK, §4.3) visits only the pages of that
 *     mask, in its order, through the page table (it jumps straight to each
 *     physical page and may take them in any order), and skips the
 *     value-side work of a block when the exact online-softmax statistics
 *     show it negligible (§3.3 Eq. (5)), with one vote per query tile
 *     (App. D.1);
 *   - dense causal prefill (§3.1; the full-attention baseline of §5.1) runs on
 *     the same kernel with every causal block visited in ascending order.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers named "device" point to GPU memory; the library never allocates
 * or frees device memory and never synchronises the host, keeps no state
 * between calls (apart from each host thread's last error message, see
 * cosa_last_error(), and the static workspace of
 * cosa_proxy_ordered_mask_no_alloc()) and enqueues all of its work on the
 * caller's stream
 * (``stream`` is a hipStream_t; NULL is the default stream).  The caller
 * owns every buffer.  Arguments are validated on the host before any
 * launch: an invalid call returns an error status and enqueues nothing.  A launch failure returns COSA_ERR_HIP.  Only host-side
 * values are checked; device contents (page ids, sequence lengths in
 * cu_seqlens) are trusted, see cosa_check_page_table_host().
 *
 * Layouts (row-major, innermost last):
 *   q, out     bf16  [total_q][num_q_heads][head_dim]   packed sequences
 *   k_pool,
 *   v_pool     bf16  [num_pages][num_kv_heads][page_size][head_dim]
 *   cu_seqlens int32 [batch+1]   prefix sums of sequence lengths (device)
 *   page_table int32 [batch][max_pages_per_seq] logical block -> page (device)
 *   lse        fp32  [num_q_heads][total_q]   natural-log sum-exp per row
 * Prefill: every sequence's query length equals its key length, the causal
 * mask admits key u for query t iff u <= t.  Grouped-query attention: query
 * head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Mask layout: "mask rows" are indexed row = (b * num_q_heads + h) * NQB + i
 * with NQB = cosa_num_q_tiles(); a mask row holds ``capacity`` int32 slots,
 * slot t at [row * capacity + t].
 *
 * Configurations that are valid but not built return COSA_ERR_UNSUPPORTED
 * (before any launch):
 *   - every entry point: head_dim other than 64 or 128; q_block other than
 *     64 or 128; page_size other than 64; kv_block other than page_size or
 *     2 * page_size; batch * num_q_heads * NQB above 2^31 - 1;
 *   - the proxy entry points (cosa_proxy_ordered_mask*, and
 *     cosa_sparse_prefill): more than 2048 logical key blocks per sequence,
 *     ceil(max_seqlen / kv_block) > 2048, i.e. max_seqlen above 131072
 *     tokens at kv_block 64 (262144 at kv_block 128); the attention entry
 *     points take sequences up to max_seqlen = 2^20;
 *   - cosa_proxy_ordered_mask_shared_kv: num_q_heads / num_kv_heads not a
 *     power of two, or (num_q_heads / num_kv_heads) * q_block / 16 > 32;
 *   - cosa_block_mask_prefill: kv_block != page_size.
 */
#ifndef COSA_H_
#define COSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  COSA_OK = 0,
  COSA_ERR_INVALID_ARG = -1, /* a host-checkable argument is out of range */
  COSA_ERR_UNSUPPORTED = -2, /* valid but not built (e.g. head_dim 96)    */
  COSA_ERR_WORKSPACE = -3,   /* workspace pointer null or too small       */
  COSA_ERR_HIP = -4          /* the HIP runtime reported a launch error    */
} cosa_status;

/* One attention layer's prefill problem.  All scalars are host values. */
typedef struct {
  int32_t batch;             /* number of sequences, >= 1                  */
  int32_t num_q_heads;       /* Hq, multiple of num_kv_heads               */
  int32_t num_kv_heads;      /* Hkv >= 1                                   */
  int32_t head_dim;          /* 64 or 128                                  */
  int32_t q_block;           /* query tile rows: 64 or 128                 */
  int32_t kv_block;          /* logical key block: page_size or 2*page_size */
  int32_t page_size;         /* tokens per KV page: 64                     */
  int32_t max_seqlen;        /* >= every sequence length, <= 1 << 20       */
  int32_t max_pages_per_seq; /* page_table row stride, >= ceil(max_seqlen / kv_block)
                                * (kv_block / page_size)                    */
  int32_t num_pages;         /* pages in the pool                          */
  int64_t total_q;           /* cu_seqlens[batch]                          */
  float softmax_scale;       /* > 0, usually 1/sqrt(head_dim)              */
  const int32_t* cu_seqlens; /* device [batch+1]                           */
  const int32_t* page_table; /* device [batch][max_pages_per_seq]          */
} cosa_problem;

/* ABI version of this header (bumped on any incompatible change). */
#define COSA_ABI_VERSION 1
int32_t cosa_abi_version(void);

/* Static text for a status code. */
const char* cosa_status_string(cosa_status status);

/* Text describing the last error returned on the calling thread ("" if none). */
const char* cosa_last_error(void);

/* Validates the host fields of ``p``.  Returns COSA_OK, COSA_ERR_INVALID_ARG
 * or COSA_ERR_UNSUPPORTED. */
cosa_status cosa_validate_problem(const cosa_problem* p);

/* NQB: query tiles of the longest sequence, ceil(max_seqlen / q_block)
 * (at least 1).  Returns a negative cosa_status on an invalid problem. */
int64_t cosa_num_q_tiles(const cosa_problem* p);

/* Mask capacity C: the largest number of blocks the KAP can keep for any
 * tile, clamp(ceil(n_max * beta), 1, n_max) with n_max = ceil(max_seqlen /
 * kv_block) and beta = floor(budget * 1e6 + 0.5) / 1e6 (integer parts per
 * million, CoSA (paperpeel) §4.1 "stage-1 budget").  budget must lie in
 * (0, 1].  Returns a negative cosa_status on error. */
int64_t cosa_mask_capacity(const cosa_problem* p, float budget);

/* Bytes of device workspace cosa_proxy_ordered_mask() needs: the pooled keys
 * as two bf16 planes (hi, lo) of [batch][num_kv_heads][n_pad][head_dim] with
 * n_pad = n_max rounded up to a multiple of 32, i.e. 4 bytes per (sequence,
 * KV head, padded key block, dim).  0 on an invalid problem. */
size_t cosa_kap_workspace_size(const cosa_problem* p);

/* Host-side check of a host copy of cu_seqlens [batch+1] and page_table
 * [batch][max_pages_per_seq]: lengths non-decreasing prefix sums ending at
 * total_q, each length <= max_seqlen, and every page id a sequence uses in
 * [0, num_pages).  Reads only host memory. */
cosa_status cosa_check_page_table_host(const cosa_problem* p, const int32_t* cu_seqlens_host,
                                       const int32_t* page_table_host);

/*
 * Kernel-Aware Proxy: ordered computation mask M_KAP (CoSA (paperpeel) §4.1,
 * §4.2 "Block ranking" / "Flag-grouped sorting", App. C.1; fused scoring and
 * pooling, §5.1 "Implementation details").
 *
 * For every mask row (sequence b, query head h, tile i of q_block rows):
 *   proxy rows: the tile's queries are pooled in groups of 16 consecutive
 *     rows (mean over the valid rows) and every key block of kv_block keys is
 *     pooled into its mean key;
 *   score s[r][j] = softmax_scale * <qbar_r, kbar_j> for the key blocks whose
 *     first key is at or before proxy row r's last query;
 *   importance w_j = mean over the tile's proxy rows of softmax_j(s[r][.]);
 *   HRM_j = j is the (lowest-index) arg-max of s[r][.] for some r;
 *   order: HRM blocks first, each group by w descending then j ascending;
 *   kept: the first k = clamp(ceil(n * beta), 1, n) entries of that order,
 *     with n the tile's candidate count (beta as in cosa_mask_capacity).
 *
 * Outputs (device, int32, per mask row; slots past the count are set to -1):
 *   ordered_blocks [rows][capacity]  logical key block ids in visiting order
 *   ordered_pages  [rows][capacity * P]  the P = kv_block / page_size pages
 *                                    of each listed block: entry t * P + s is
 *                                    page_table[b][ordered_blocks[t] * P + s],
 *                                    -1 for a page past the sequence's end
 *                                    (a logical block resolved through one or
 *                                    more physical pages, pp App. D.1)
 *   counts         [rows]            k (0 for tiles past a sequence's end)
 *   hrm_counts     [rows] nullable   number of HRM blocks among the kept ones
 *                                    (they are its first hrm_counts slots)
 *   debug_w        [rows][n_max] nullable fp32 importance w_j (0 past n)
 *   debug_hrm      [rows][n_max] nullable uint8 HRM flags
 * ``capacity`` must be >= cosa_mask_capacity(p, budget).  ``workspace`` must
 * hold cosa_kap_workspace_size(p) bytes (device, any contents).
 * COSA_ERR_UNSUPPORTED when ceil(max_seqlen / kv_block) > 2048 (the whole
 * candidate list of a tile is scored and selected in one pass).
 */
cosa_status cosa_proxy_ordered_mask(const cosa_problem* p, const void* q, const void* k_pool,
                                    float budget, int32_t* ordered_blocks,
                                    int32_t* ordered_pages, int32_t* counts,
                                    int32_t* hrm_counts, float* debug_w, uint8_t* debug_hrm,
                                    int64_t capacity, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and outputs as cosa_proxy_ordered_mask(), bit for bit, with
 * the pooled-key workspace held in a static device array of the library
 * instead of a caller's buffer.  Every GPU the library runs on holds its own
 * COSA_NO_ALLOC_SCRATCH_BYTES copy until the process ends; its device
 * address is looked up once per device (hipGetSymbolAddress) on the first
 * call there.  The call allocates nothing, device or host.
 *
 * Limit: problems with cosa_kap_workspace_size(p) >
 * COSA_NO_ALLOC_SCRATCH_BYTES (32 MiB: four 128K sequences with 8 KV heads
 * of head_dim 128) return COSA_ERR_WORKSPACE before any launch.  The array
 * keeps the last call's contents between calls and every call on a GPU uses
 * the same array, so calls that overlap on one GPU (on different streams)
 * race; a call needs no zeroed array (the proxy writes every pooled key it
 * reads).  Other arguments and errors as for cosa_proxy_ordered_mask();
 * COSA_ERR_HIP if the stream's device cannot be queried.
 */
#define COSA_NO_ALLOC_SCRATCH_BYTES (32u << 20)
cosa_status cosa_proxy_ordered_mask_no_alloc(const cosa_problem* p, const void* q,
                                             const void* k_pool, float budget,
                                             int32_t* ordered_blocks, int32_t* ordered_pages,
                                             int32_t* counts, int32_t* hrm_counts,
                                             float* debug_w, uint8_t* debug_hrm,
                                             int64_t capacity, void* stream);

/*
 * Kernel-Aware Proxy with stage-1 Top-p (CoSA (paperpeel) §5.1
 * "Hyperparameters" and App. D.1: Top-p selection, p = 0.95 for Qwen3-8B).
 *
 * As cosa_proxy_ordered_mask(), except that the kept count of a tile is
 *   k = min(budget count, Top-p count),
 * the Top-p count being the smallest k >= 1 such that the first k blocks of
 * the HRM-first order carry at least the mass p, where the mass of a block
 * is its importance w_j (the w_j of a tile sum to 1).  The sum is taken
 * exactly in fixed point: every w_j (the fp32 value debug_w reports) is
 * rounded down to a multiple of 2^-48 and p to floor(p * 2^48) * 2^-48, so
 * the count depends on neither summation order nor run.  top_p = 1 keeps
 * every candidate the budget allows; if the masses never reach p, likewise.
 * top_p must lie in (0, 1]; budget (the cap, 1 for none) and capacity as for
 * cosa_proxy_ordered_mask().
 */
cosa_status cosa_proxy_ordered_mask_top_p(const cosa_problem* p, const void* q,
                                          const void* k_pool, float top_p, float budget,
                                          int32_t* ordered_blocks, int32_t* ordered_pages,
                                          int32_t* counts, int32_t* hrm_counts, float* debug_w,
                                          uint8_t* debug_hrm, int64_t capacity, void* workspace,
                                          size_t workspace_bytes, void* stream);

/*
 * Kernel-Aware Proxy with one mask per KV head, shared by the query heads that
 * read it (grouped-query attention; the pages leave the packing of a KV
 * group to the implementation, pp §4.3 / App. D.1 name only the per-tile
 * mask).  For mask row (b, g, i) the proxy rows of tile i of every query
 * head h with h / (num_q_heads / num_kv_heads) == g are scored together
 * against the pooled keys of KV head g: w_j is the mean over all of them of
 * their per-row softmax, HRM_j marks the arg-max block of any of them; order,
 * budget and remap as for cosa_proxy_ordered_mask().  top_p in (0, 1] as for
 * cosa_proxy_ordered_mask_top_p() (1 = budget only).
 *
 * Mask arrays are laid out per KV head: ordered_blocks / ordered_pages
 * [batch][num_kv_heads][NQB][capacity], counts / hrm_counts
 * [batch][num_kv_heads][NQB], debug_w / debug_hrm [..][NQB][n_max].
 * Requires (num_q_heads / num_kv_heads) a power of two with
 * (num_q_heads / num_kv_heads) * q_block / 16 <= 32 (COSA_ERR_UNSUPPORTED
 * otherwise); with one query head per KV head it equals the per-head mask.
 */
cosa_status cosa_proxy_ordered_mask_shared_kv(const cosa_problem* p, const void* q,
                                              const void* k_pool, float top_p, float budget,
                                              int32_t* ordered_blocks, int32_t* ordered_pages,
                                              int32_t* counts, int32_t* hrm_counts,
                                              float* debug_w, uint8_t* debug_hrm,
                                              int64_t capacity, void* workspace,
                                              size_t workspace_bytes, void* stream);

/*
 * Ordered-Skipping Kernel (CoSA (paperpeel) §4.3, App. D.1; skip rule §3.3).
 *
 * For every mask row (b, h, i) the kernel walks slots t = 0..counts[row]-1 in
 * order, fetching the key/value pages ordered_pages[row][t * P .. t * P + P-1]
 * (P = kv_block / page_size; the pages of logical block
 * ordered_blocks[row][t], which gives the causal mask), forms the exact logits
 * S = softmax_scale * Q K^T of the tile, and keeps the online-softmax running
 * max m and sum l per query row.  If skip_tau >= 0 and every valid row r of
 * the tile has max_c S[r][c] < m_r - skip_tau (the running max before the
 * block; -inf < -inf is false), the block's value side (softmax weights,
 * l and O updates, the V page read from LDS) is skipped.  skip_tau < 0 turns
 * the skip off (Delta = -1 in App. D.1).  Blocks may come in any order (the
 * result of online softmax does not depend on it, §3.2).
 *
 * out        device bf16 [total_q][Hq][D]: softmax-weighted values over the
 *            computed keys; 0 for a row that saw no key.
 * lse        device fp32 [Hq][total_q] nullable: log-sum-exp (natural log)
 *            over the computed keys, -inf for a row that saw no key.
 * skip_record device uint8 [rows][capacity] nullable: 1 if slot t was
 *            skipped in-kernel, 0 if computed; slots past the count untouched.
 * row_stats  device int32 [rows][2] nullable: (visited slots, skipped slots).
 * Every listed block id must lie in [0, ceil(L_b / kv_block)) for its
 * sequence and every page id of a page holding keys of the sequence in
 * [0, num_pages); counts[row] must lie in [0, min(capacity, the number of
 * logical blocks the tile's last row sees)], which is at most 16384 (the
 * kernel keeps one skip bit per slot of a tile in LDS and does not check).  With kv_block = 2 * page_size the vote and the skip cover
 * the whole 128-key logical block (the pages' b = 128, App. D.1).
 */
cosa_status cosa_osk_prefill(const cosa_problem* p, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* ordered_blocks,
                             const int32_t* ordered_pages, const int32_t* counts,
                             int64_t capacity, float skip_tau, void* out, float* lse,
                             uint8_t* skip_record, int32_t* row_stats, void* stream);

/*
 * The proxy and the Ordered-Skipping Kernel in one call (CoSA (paperpeel)
 * §4.1: KAP emits the ordered mask that the OSK consumes).  Same result, bit
 * for bit, as cosa_proxy_ordered_mask() followed by cosa_osk_prefill() with
 * these arguments (debug_w and debug_hrm not available): the masks are
 * written to ordered_blocks / ordered_pages / counts / hrm_counts and the
 * attention to out / lse / skip_record / row_stats, with the layouts given
 * there.
 *
 * The work is cut into at most 8 chunks of (sequence, KV head) groups, each
 * chunk's kernel at least 8192 workgroups (query heads x query tiles) where
 * the groups allow, so short inputs run as one chunk; the proxy of every
 * chunk runs on `stream`.  With aux_stream != NULL (another stream of the
 * same device, not `stream`) and more than one chunk, the kernel of chunk c
 * runs on aux_stream after the proxy of chunk c, so that the proxy of later
 * chunks overlaps it, and `stream` waits for the last kernel before the
 * call's later work; otherwise everything runs on `stream` in chunk order.  Argument errors (including the proxy's 2048-key-block limit) as
 * for the two calls; COSA_ERR_HIP if an event cannot be created.  The call
 * allocates no device memory.
 */
cosa_status cosa_sparse_prefill(const cosa_problem* p, const void* q, const void* k_pool,
                                const void* v_pool, float budget, float skip_tau,
                                int32_t* ordered_blocks, int32_t* ordered_pages, int32_t* counts,
                                int32_t* hrm_counts, int64_t capacity, void* workspace,
                                size_t workspace_bytes, void* out, float* lse,
                                uint8_t* skip_record, int32_t* row_stats, void* stream,
                                void* aux_stream);

/*
 * Ordered-Skipping Kernel over masks shared per KV head (the layout of
 * cosa_proxy_ordered_mask_shared_kv()): query head h of sequence b, tile i
 * walks mask row (b, h / (num_q_heads / num_kv_heads), i).  Everything else,
 * including the per-head, per-tile skip vote and the per-head skip_record /
 * row_stats layout [batch][num_q_heads][NQB](...), is as for
 * cosa_osk_prefill().  The query heads of one KV head run side by side on one
 * XCD so that the pages they share are fetched into its L2 once.
 */
cosa_status cosa_osk_prefill_shared_kv(const cosa_problem* p, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* ordered_blocks,
                                       const int32_t* ordered_pages, const int32_t* counts,
                                       int64_t capacity, float skip_tau, void* out, float* lse,
                                       uint8_t* skip_record, int32_t* row_stats, void* stream);

/*
 * Ordered-Skipping Kernel with the length-adaptive threshold Delta / N
 * (CoSA (paperpeel) §5.1 "Hyperparameters", App. D.1: Delta = 2000 for
 * Qwen3-8B, 200 for Llama-3.1-8B, Delta = -1 disables the skip).
 *
 * As cosa_osk_prefill(), with the threshold of sequence b of L_b tokens
 * tau_b = ln(L_b / skip_delta) nats (Delta / N read as the bound on
 * exp(block max - running max)).  skip_delta > 0 turns the skip on whatever
 * the sign of tau_b (a sequence shorter than Delta then keeps only blocks
 * that raise some row's max); skip_delta <= 0 turns it off.  skip_delta must
 * be finite.
 */
cosa_status cosa_osk_prefill_delta(const cosa_problem* p, const void* q, const void* k_pool,
                                   const void* v_pool, const int32_t* ordered_blocks,
                                   const int32_t* ordered_pages, const int32_t* counts,
                                   int64_t capacity, float skip_delta, void* out, float* lse,
                                   uint8_t* skip_record, int32_t* row_stats, void* stream);

/*
 * Dense causal prefill on the same page step: every tile visits all of its
 * causal keys in ascending order through page_table, one page_size-key page at
 * a time whatever kv_block is (the result does not depend on the logical block
 * size), with no in-kernel skip (CoSA (paperpeel) §3.1, FlashAttention-2
 * baseline of §5.1).  out / lse as for cosa_osk_prefill().
 */
cosa_status cosa_dense_prefill(const cosa_problem* p, const void* q, const void* k_pool,
                               const void* v_pool, void* out, float* lse, void* stream);

/*
 * Logical mask skipping on the same kernel, the comparison point of the
 * kernel microbenchmark of CoSA (paperpeel) App. D.3, Fig. B (and §4.3): a
 * block-sparse kernel driven by a binary block mask walks every causal block
 * of a tile in ascending order and computes only the selected ones, paying
 * the loop control and the per-block workgroup barrier on the unselected
 * ones too, whereas the OSK jumps straight to the pages of its ordered list.
 * No in-kernel skip.
 *
 * block_mask  device uint32 [rows][mask_words]: bit (j % 32) of word j / 32
 *             of mask row (b, h, i) selects causal key block j of that tile;
 *             bits at or past the tile's causal block count are ignored.
 * mask_words  >= ceil(ceil(max_seqlen / kv_block) / 32).
 * out / lse as for cosa_osk_prefill(), over the selected blocks.
 */
cosa_status cosa_block_mask_prefill(const cosa_problem* p, const void* q, const void* k_pool,
                                    const void* v_pool, const uint32_t* block_mask,
                                    int64_t mask_words, void* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* COSA_H_ */
