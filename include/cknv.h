/*
 * cknv.h -- C ABI of the CompKV block-sparse decode step for AMD MI355X (gfx950).
 *
 * One decode step of one attention layer, for S sequences that each have H KV
 * heads shared by G query heads (GQA), runs as
 *
 *   cknv_append        add the step's token, refresh its block's summary
 *   cknv_score_select  score every block, keep the forced set + Top-K
 *   cknv_attend        exact attention over kept blocks + Mean compensation
 *
 * or as one call, cknv_decode_step, which fuses the three.
 *
 * Method: the CompKV page (onedev.kr/papers/157). Section names cited below:
 *   "How it works"  -- Mean compensation, GQA group, budget of K blocks;
 *   "What differs"  -- block summary, estimators z̄, σ̂², p̂, S_b, forced set,
 *                      Top-K, joint normalisation;
 *   "How to use it" -- per-step update of the current block's statistics;
 *                      BF16 KV cache with FP32 summaries;
 *   "Assumptions and limits" -- block size 16, default r = 4.
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer owned by the caller, except the
 *     cknv_shape / cknv_cache structs themselves (host memory, read during
 *     the call only) and the out-parameters of cknv_workspace_size and
 *     cknv_kv_placement. The KV and summary arrays of a cknv_cache may
 *     instead be pinned host memory that the device reads and writes at
 *     the same address (the host-offload placement, see cknv_kv_placement).
 *     The library never allocates, frees or synchronises.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *     asynchronously; results are ready when the stream reaches them.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     validation error nothing is enqueued and no HIP call is made.
 *     Return value: CKNV_OK or a negative status (cknv_status_str names it).
 *   - A unit is one (sequence s, KV head h), index u = s*H + h. Query head
 *     g of unit u is row u*G + g of q and out (consecutive query heads share
 *     a KV head).
 *   - Token t of a unit lives in block t/16, slot t%16. The number of
 *     blocks of a unit is NB = ceil(seq_len[s] / 16); the last block may be
 *     partial (the open block).
 *   - Calls that share one workspace must not overlap (same stream, in
 *     order). cknv_attend consumes what cknv_score_select left in it.
 */
#ifndef CKNV_H
#define CKNV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CKNV_OK 0
#define CKNV_EINVAL (-1)        /* null pointer, non-positive or inconsistent size */
#define CKNV_EUNSUPPORTED (-2)  /* d not 64/128, G not 1/2/4/8, block != 16, r not dividing d, unknown flags, or too many blocks */

/* cknv_shape.flags: the ablation variants the page reports ("Assumptions and
 * limits"); 0 is CompKV itself. Any combination is allowed. */
#define CKNV_FLAG_NO_COMPENSATION 0x1u  /* unselected blocks are dropped instead of Mean-compensated */
#define CKNV_FLAG_MASS_ONLY_SCORE 0x2u  /* S_b = sum_g p̂_{g,b}: no outer variance factor */
#define CKNV_FLAG_FIRST_ORDER_MASS 0x4u /* p̂ from |b| exp(z̄): no σ̂²/2 in the mass estimate */
#define CKNV_FLAGS_ALL 0x7u
#define CKNV_ENOSPACE (-3)      /* workspace smaller than cknv_workspace_size, or max_blocks > cap_blocks */
#define CKNV_EHIP (-4)          /* a HIP call or kernel launch failed */

/* Size of the per-GPU device array cknv_decode_step_noalloc works in. */
#define CKNV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* Problem shape. */
typedef struct cknv_shape {
  int32_t S;          /* sequences */
  int32_t H;          /* KV heads per sequence */
  int32_t G;          /* query heads per KV head (GQA group), 1, 2, 4 or 8 */
  int32_t d;          /* head dimension, 64 or 128 */
  int32_t r;          /* variance groups of the key coordinates, divides d */
  int32_t block;      /* tokens per block, must be 16 */
  int32_t cap_blocks; /* capacity of every unit, in blocks */
  uint32_t flags;     /* 0, or CKNV_FLAG_* bits (ablation variants) */
} cknv_shape;

/* KV cache and block-summary store of one layer, all in HBM (device pointers).
 * Summary of block b of unit u ("What differs": {|b|, k̄_b, D̄_b, v̄_b},
 * 2d + r + 1 FP32 scalars per block, kept as four arrays):
 *   kbar[(u*cap_blocks + b)*d + i]  mean key, coordinate i
 *   dbar[(u*cap_blocks + b)*r + t]  mean over i in group t of the population
 *                                    variance of key coordinate i; group t is
 *                                    coordinates [t*d/r, (t+1)*d/r)
 *   cnt [u*cap_blocks + b]           |b|, tokens in the block (1..16)
 *   vbar[(u*cap_blocks + b)*d + i]  mean value, coordinate i
 * Tokens ("How to use it": BF16 KV cache):
 *   k[(u*cap_blocks*16 + t)*d + i], v[...] bfloat16 bit patterns.
 * seq_len[s]: tokens held by sequence s (all its heads), device-resident so
 * a step can be replayed from a HIP graph. */
typedef struct cknv_cache {
  uint16_t* k;
  uint16_t* v;
  float* kbar;
  float* dbar;
  float* cnt;
  float* vbar;
  int32_t* seq_len;
} cknv_cache;

/* Bytes of workspace the score/select, attend and dense calls need for this
 * shape, max_blocks and budget. Host-only; makes no HIP call.
 * max_blocks: upper bound on NB over all sequences for the calls that will
 * use the workspace (the kernels' grid is sized by it).
 * budget_tokens: the token budget those calls will pass. */
int cknv_workspace_size(const cknv_shape* shape, int32_t max_blocks, int32_t budget_tokens,
                        size_t* bytes);

/* Zero-fill the workspace. Optional: every call writes the workspace
 * regions it reads before reading them. Enqueues a kernel (no memset), so
 * it may be captured in a graph. */
int cknv_workspace_init(const cknv_shape* shape, int32_t max_blocks, int32_t budget_tokens,
                        void* ws, size_t ws_bytes, void* stream);

/* Append one token to every unit and refresh the summary of the block it
 * lands in ("How to use it": a fused kernel updates the current block's
 * statistics and stores the new K/V every step). The block's summary is
 * recomputed from its (up to 16) tokens in FP32, two-pass (mean, then
 * population variance). Afterwards seq_len[s] += 1 for every sequence.
 * new_k, new_v: bfloat16 [S][H][d]. A sequence whose cache is full
 * (seq_len == 16*cap_blocks) is left unchanged. Needs no workspace. */
int cknv_append(const cknv_shape* shape, const cknv_cache* cache, const uint16_t* new_k,
                const uint16_t* new_v, void* stream);

/* Build the summary of every block of every unit from the cache (blocks
 * 0..NB-1, NB from seq_len). Same arithmetic as cknv_append. Used after a
 * prefill; also rebuilds the store from the cache. */
int cknv_build_summaries(const cknv_shape* shape, const cknv_cache* cache, int32_t max_blocks,
                         void* stream);

/* Score every block of every unit and select the kept blocks.
 * Scores ("What differs"), for query head g of the unit and block b:
 *   z̄_{g,b}  = q_g . k̄_b / sqrt(d)
 *   σ̂²_{g,b} = (1/d) sum_t (sum_{i in group t} q_{g,i}^2) D̄_{b,t}
 *   p̂_{g,b}  = |b| exp(z̄ + σ̂²/2) / sum over all blocks c of the unit of the same
 *   S_b      = sum_g p̂_{g,b} σ̂²_{g,b}
 * Selection ("What differs"): Kb = budget_tokens/16 block slots (Kb >= 3). If
 * NB <= Kb every block is kept; else the first block and the last two are
 * always kept and the other Kb-3 slots go to the largest S_b, ties to the
 * lower block index.
 * q: fp32 [S][H*G][d]. Outputs: sel [S*H][Kb] (kept block indices,
 * ascending, first n_sel[u] entries valid), n_sel [S*H] = min(Kb, NB);
 * scores [S*H][cap_blocks] (S_b of blocks 0..NB-1, fp32) or NULL.
 * Also leaves in the workspace the per-chunk Mean-compensation sums that
 * cknv_attend consumes. Blocks at or beyond max_blocks are ignored. */
int cknv_score_select(const cknv_shape* shape, const cknv_cache* cache, const float* q,
                      int32_t budget_tokens, int32_t max_blocks, float* scores, int32_t* sel,
                      int32_t* n_sel, void* ws, size_t ws_bytes, void* stream);

/* Attention output of every query head ("How it works", "What differs"):
 * kept blocks contribute their tokens' exact softmax terms; every other
 * block contributes Mean compensation, |b| exp(z̄_{g,b}) to the normaliser
 * and |b| exp(z̄_{g,b}) v̄_b to the value sum; one shared normaliser:
 *   out_g = [sum_kept sum_i e^{z_i} v_i + sum_other |b| e^{z̄_b} v̄_b]
 *         / [sum_kept sum_i e^{z_i}     + sum_other |b| e^{z̄_b}]
 * with z_i = q_g . k_i / sqrt(d). lse_g = log of that denominator.
 * Must follow cknv_score_select on the same workspace with the same q,
 * budget_tokens and max_blocks. sel / n_sel: as written by it, or any other
 * list of n_sel[u] <= Kb DISTINCT block indices < NB per unit (entries
 * outside [0, NB) are ignored).
 * out: fp32 [S][H*G][d]; lse: fp32 [S][H*G] or NULL. A unit with NB = 0 gets
 * out = 0, lse = -inf. */
int cknv_attend(const cknv_shape* shape, const cknv_cache* cache, const float* q,
                const int32_t* sel, const int32_t* n_sel, int32_t budget_tokens,
                int32_t max_blocks, float* out, float* lse, void* ws, size_t ws_bytes,
                void* stream);

/* One whole decode step, fused: the same results as cknv_append, then
 * cknv_score_select, then cknv_attend on the same arguments, in two kernel
 * launches instead of five.
 *   - new_k, new_v: bfloat16 [S][H][d], the step's token ("How to use it":
 *     the new K/V are stored and the current block's statistics refreshed);
 *   - q, budget_tokens, scores, sel, n_sel: as for cknv_score_select, with
 *     NB counted after the append; out, lse: as for cknv_attend.
 * max_blocks bounds NB after the append. seq_len[s] advances by one for
 * every sequence whose cache has room (a full cache is left unchanged and
 * the step attends its existing tokens; so is a sequence whose token would
 * land at or past block max_blocks, which breaks the bound). The workspace regions are those of
 * cknv_score_select / cknv_attend plus the step's own. */
int cknv_decode_step(const cknv_shape* shape, const cknv_cache* cache, const uint16_t* new_k,
                     const uint16_t* new_v, const float* q, int32_t budget_tokens,
                     int32_t max_blocks, float* scores, int32_t* sel, int32_t* n_sel, float* out,
                     float* lse, void* ws, size_t ws_bytes, void* stream);

/* The two halves of cknv_decode_step, for callers that schedule them apart
 * (call them in this order on one workspace, with nothing that changes the
 * cache or seq_len in between):
 *   cknv_decode_score   the append of the step's token and the summary of
 *                       the block it lands in, and the streaming pass over
 *                       the summaries of the blocks closed before the token
 *                       (scores' ingredients and the Mean-compensation sums
 *                       of every one of them); records seq_len in the
 *                       workspace and leaves it unchanged;
 *   cknv_decode_finish  the normalisers, the selection, and the attention
 *                       with compensation; advances seq_len.
 * Arguments as for cknv_decode_step. */
int cknv_decode_score(const cknv_shape* shape, const cknv_cache* cache, const uint16_t* new_k,
                      const uint16_t* new_v, const float* q, int32_t budget_tokens,
                      int32_t max_blocks, void* ws, size_t ws_bytes, void* stream);
int cknv_decode_finish(const cknv_shape* shape, const cknv_cache* cache, const float* q,
                       int32_t budget_tokens, int32_t max_blocks, float* scores, int32_t* sel,
                       int32_t* n_sel, float* out, float* lse, void* ws, size_t ws_bytes,
                       void* stream);

/* Where a cache's arrays live, checked before any of them is used on the
 * device. The page keeps the BF16 KV cache and the FP32 summaries in pinned
 * CPU memory and moves what a step needs over the host link ("How to use
 * it"); here every entry point also accepts k and v, and the four summary
 * arrays, in pinned host memory (hipHostMalloc, as torch's pin_memory
 * allocates it) mapped for the current device at the same address: the
 * kernels then read the kept blocks' tokens (and the summaries) through the
 * host link and write the step's token there, with no host round trip.
 * On CKNV_OK, *placement = CKNV_KV_ON_HOST if k and v are such host memory
 * (0: device memory of the current device), plus CKNV_SUMMARIES_ON_HOST
 * if kbar, dbar, cnt and vbar are. Host-only: HIP pointer queries, no
 * enqueue.
 * Errors: CKNV_EINVAL if a pointer is null, k and v (or the four summary
 * arrays) are placed differently, an array is pageable host memory, device
 * memory of another device, or host memory the device sees at another
 * address, or seq_len is not device memory; CKNV_EHIP if the runtime
 * cannot be queried (no device). */
#define CKNV_KV_ON_HOST 0x1
#define CKNV_SUMMARIES_ON_HOST 0x2
int cknv_kv_placement(const cknv_shape* shape, const cknv_cache* cache, int32_t* placement);

/* Full (dense) softmax attention over every cached token, the baseline the
 * page compares CompKV with ("Assumptions and limits"). Same q/out/lse
 * layouts as cknv_attend. Uses its own region of the workspace. */
int cknv_dense_attend(const cknv_shape* shape, const cknv_cache* cache, const float* q,
                      int32_t budget_tokens, int32_t max_blocks, float* out, float* lse,
                      void* ws, size_t ws_bytes, void* stream);

/* cknv_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that forbid allocation): the same
 * arguments and results without `ws`/`ws_bytes`. Its workspace is a
 * library-owned device array of CKNV_NOALLOC_SCRATCH_BYTES (32 MiB), one per
 * GPU, held until the process ends; the call itself allocates and
 * frees nothing. A shape, max_blocks and budget whose workspace
 * (cknv_workspace_size) exceeds it return CKNV_ENOSPACE with nothing
 * enqueued. Every call on a GPU shares that GPU's array, so calls that
 * overlap on one GPU (other streams, other host threads) race: issue them
 * in order on one stream. When the workspace layout changes from the
 * previous call on the device, the call first clears the step counters with
 * a kernel (no memset). */
int cknv_decode_step_noalloc(const cknv_shape* shape, const cknv_cache* cache,
                             const uint16_t* new_k, const uint16_t* new_v, const float* q,
                             int32_t budget_tokens, int32_t max_blocks, float* scores,
                             int32_t* sel, int32_t* n_sel, float* out, float* lse, void* stream);

/* Name of a status code (static string). */
const char* cknv_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* CKNV_H */
