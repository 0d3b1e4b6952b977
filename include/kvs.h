/*
 * kvs.h -- attention-space KV-cache scoring and budgeted top-k on AMD MI355X
 * (gfx950).  Plain C ABI: device pointers, sizes and a HIP stream handle.
 *
 * Two modes share the library:
 *   - IntentKV ("Cross-turn intent-aware KV cache pruning for multi-turn
 *     reasoning agents"): QueryMemory rule scoring (Sec. 3.2, Eqs. 2-4),
 *     budgeted top-k with a forced set (Sec. 3.1, Eq. 1), and eviction by
 *     redirecting dropped slots to a dead slot (abstract, Sec. 1, Sec. 3).
 *   - KVMEM ("Virtualising million-token agent workspaces onto a laptop
 *     GPU"): Mean-K block index and block relevance R_b (section "Design and
 *     trade-offs: step-level attention trigger and Mean-K model-native
 *     retrieval"), and the execution view rebuilt by re-applying RoPE to raw K
 *     at compact page-table positions (section "Engineering and cost: tiered
 *     movement, page-table aliasing and position-consistent reconstruction").
 *
 * Conventions for every call
 *   - Tensors are caller-owned, contiguous, row-major device buffers in the
 *     layout stated per argument.  The library never allocates, frees or keeps
 *     a pointer after the call returns.  Scratch memory is a caller workspace
 *     whose size comes from the matching *_workspace() query; the one
 *     exception, kvs_topk_select_noalloc, uses a fixed static device array of
 *     the library instead.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work on it and return without synchronising.
 *   - The return value is a kvs_status, decided on the host before any work is
 *     enqueued (argument and shape checks).  A failed launch returns
 *     KVS_ERR_HIP.  Nothing is thrown across the ABI.
 *   - Results are deterministic: identical inputs give identical bits (no
 *     floating-point atomics; fixed reduction orders).
 *   - Layouts use the pages' notation: L layers, H_q query heads, H_kv KV
 *     heads (G = H_q / H_kv query heads share KV head g = h / G), D head
 *     dimension, N tokens.
 *   - bf16 means IEEE binary32 with the low 16 bits dropped (uint16 storage).
 *   - A data pointer may be NULL only where its tensor holds no elements.
 *   - Sizes that would need a launch of 2^24 or more workgroups (far beyond
 *     any single-GPU cache) return KVS_ERR_SHAPE.
 */
#ifndef KVS_H_
#define KVS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvs_status;

#define KVS_OK 0
#define KVS_ERR_ARG 1          /* null pointer, negative size, bad range, non-finite scalar */
#define KVS_ERR_SHAPE 2        /* inconsistent sizes (H_q % H_kv != 0, size overflow, ...) */
#define KVS_ERR_DTYPE 3        /* dtype code not accepted by this call */
#define KVS_ERR_UNSUPPORTED 4  /* valid but not built: D outside {64, 128}, block != 32 */
#define KVS_ERR_WORKSPACE 5    /* workspace missing or smaller than the query says */
#define KVS_ERR_HIP 6          /* the HIP runtime rejected a launch */
#define KVS_ERR_LIMIT 7        /* size above the fixed limit of a no-allocation entry point */

#define KVS_F32 0
#define KVS_BF16 1

/* Human-readable name of a status code (static string). */
const char* kvs_status_string(kvs_status s);

/* Library version, as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t kvs_version(void);

/*
 * QueryMemory update -- IntentKV Sec. 3.2, Eq. (2).
 *   M <- exp(-lambda) * M + Enc(q_t);  M[l,h,:] <- M[l,h,:] / ||M[l,h,:]||_2
 * Enc(q_t) is the mean of the S post-RoPE query rows of the actionable span.
 *   q_span   [L, H_q, S, D], dtype q_dtype (KVS_F32 or KVS_BF16), device.
 *   lambda   decay rate >= 0; +INFINITY gives the page's "query" mode.
 *   first_turn  nonzero: the previous M is taken as zero and M is not read.
 *   M        [L, H_q, D] float32, device, read (unless first_turn) and written.
 * A zero vector stays zero.  Errors: KVS_ERR_ARG (null, S < 1, lambda < 0 or
 * NaN), KVS_ERR_DTYPE, KVS_ERR_UNSUPPORTED (D not 64 or 128).
 */
kvs_status kvs_qmem_update(const void* q_span, int32_t q_dtype, int32_t L, int32_t H_q,
                           int32_t S, int32_t D, float lambda, int32_t first_turn, float* M,
                           void* stream);

/* Workspace bytes kvs_rule_score needs for these sizes. */
size_t kvs_rule_score_workspace(int32_t L, int32_t H_q, int32_t H_kv, int64_t N);

/*
 * Rule score -- IntentKV Sec. 3.2, Eqs. (3)-(4), with the candidate set of
 * Sec. 3.1.  For every layer l and query head h, a softmax over the candidate
 * positions H = [0,N) \ F of M[l,h] . K[l,h/G,j] / sqrt(D), summed over
 * (l, h):  rule[j] = sum_{l,h} a_{l,h,j}.  F = [0,pi) U [q_s,q_e).
 *   K        [L, H_kv, N, D] post-RoPE keys, dtype k_dtype (KVS_F32 or KVS_BF16).
 *   M        [L, H_q, D] float32 QueryMemory.
 *   pi       protected prefix length (clipped to N); q_s <= q_e actionable span.
 *   rule     [N] float32 output; exactly 0 on F.  sum(rule) = L*H_q when H is
 *            non-empty.
 *   ws       device workspace of >= kvs_rule_score_workspace() bytes.
 * Errors: KVS_ERR_ARG, KVS_ERR_SHAPE (H_q % H_kv, N > 2^31-1), KVS_ERR_DTYPE,
 * KVS_ERR_UNSUPPORTED (D not 64/128), KVS_ERR_WORKSPACE.
 */
kvs_status kvs_rule_score(const void* K, int32_t k_dtype, const float* M, int32_t L,
                          int32_t H_q, int32_t H_kv, int32_t D, int64_t N, int64_t pi,
                          int64_t q_s, int64_t q_e, float* rule, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * Rule score reading K in place from a paged pool -- IntentKV Sec. 3.1
 * (slot map S_r of the request) and the layout layer of the abstract and
 * Sec. 1 (SGLang/vLLM paged caches; survivors keep their slot).  Same result
 * as kvs_rule_score on K[l,g,j,:] = K_pool[l, slots[j], g, :], with one more
 * rule: a position whose slot lies outside [0, pool_size) -- the dead slot
 * of an earlier eviction -- has no key, so it drops out of every softmax like
 * a forced position and scores 0.
 *   K_pool   [L, pool_size, H_kv, D] token-major pool, dtype k_dtype.
 *   slots    [N] int64 slot map (device).
 *   ws       device workspace of >= kvs_rule_score_workspace(L, H_q, H_kv, N) bytes.
 * Other arguments and errors as kvs_rule_score (pool_size < 1 -> KVS_ERR_ARG).
 */
kvs_status kvs_rule_score_paged(const void* K_pool, int32_t k_dtype, const int64_t* slots,
                                int64_t pool_size, const float* M, int32_t L, int32_t H_q,
                                int32_t H_kv, int32_t D, int64_t N, int64_t pi, int64_t q_s,
                                int64_t q_e, float* rule, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * Bounded wait of the rule scorer's fold -- a diagnostic and test setting;
 * the default suits every size.  With bf16 keys and G <= 8 both rule-score
 * calls run as a work queue: a workgroup keeps a chunk's logits on chip and
 * folds its G heads into one value per position once every chunk of its
 * (layer, KV head) group has published its softmax partials.  A chunk whose
 * group is not complete when its workgroup gets to it is spilled and summed
 * by the column pass instead, with the same bits as a result.  polls >= 0:
 * the one blocking wait (at the end, once every chunk is claimed) polls at
 * most that often before it spills; polls < 0: no chunk is folded.
 * Process-wide, for calls launched after it returns.  Returns the previous
 * value.
 */
int64_t kvs_rule_score_wait_limit(int64_t polls);

/* Workspace bytes kvs_window_score needs for these sizes. */
size_t kvs_window_score_workspace(int32_t L, int32_t H_q, int32_t H_kv, int64_t W, int64_t N);

/*
 * Window score -- the SnapKV-style window of W tail query rows that IntentKV
 * Sec. 3.2 says Eq. (3) replaces with one accumulated query state: for every
 * layer l, query head h and window row w a softmax over the candidate
 * positions H = [0,N) minus F (Sec. 3.1) of Qw[l,h,w] . K[l,h/G,j] / sqrt(D),
 * summed over (l, h, w):  score_j = sum_{l,h,w} a_{l,h,w,j}.  With W = 1 and
 * Qw = M this is kvs_rule_score.  SnapKV's pooling and per-head selection are
 * not part of it.
 *   K        [L, H_kv, N, D] bf16 post-RoPE keys.
 *   Qw       [L, H_q, W, D] bf16 post-RoPE window query rows.
 *   score    [N] float32 output; 0 on F; sum over H = L*H_q*W.
 *   ws       device workspace of >= kvs_window_score_workspace() bytes.
 * Errors: KVS_ERR_ARG (null, W < 1, bad range), KVS_ERR_SHAPE (also N or
 * G*W at or above 2^23 - 128 rows), KVS_ERR_UNSUPPORTED (D not 64/128),
 * KVS_ERR_WORKSPACE.
 */
kvs_status kvs_window_score(const void* K, const void* Qw, int32_t L, int32_t H_q, int32_t H_kv,
                            int32_t D, int64_t N, int64_t W, int64_t pi, int64_t q_s, int64_t q_e,
                            float* score, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes kvs_topk_select uses for n scores: 0 up to 32768 scores;
 * beyond that a few KB that select the multi-workgroup path (ws may also be
 * NULL there, for a slower single-workgroup selection that needs none). */
size_t kvs_topk_workspace(int64_t n);

/*
 * Budgeted top-k with a forced set -- IntentKV Sec. 3.1, Eq. (1); KVMEM's
 * "sink and recent blocks are always kept, the rest of the budget goes to the
 * largest R_b" is the same call with the sink and recent ranges as forced.
 *   score    [n] float32 scores.
 *   [f0_begin, f0_end), [f1_begin, f1_end)  forced ranges (clipped, may overlap).
 *   C        total budget including the forced positions; C* = max(0, C - |F|).
 *   keep_mask [n] uint8 output: 1 = kept.
 *   keep_idx  [n] int32 output: kept indices ascending in the first n_kept
 *             entries; the rest is left untouched.
 *   n_kept    device int64 output: |F| + min(C*, n - |F|).
 * Order among candidates: larger score first; equal scores -> lower index
 * first (Eq. 1's argmax is not unique under ties); NaN below every number;
 * -0.0 equal to +0.0.  C >= n keeps everything; C < |F| keeps F only.
 *   ws        device workspace of kvs_topk_workspace(n) bytes, or NULL (see there).
 * Errors: KVS_ERR_ARG, KVS_ERR_SHAPE (n > 2^31-1), KVS_ERR_WORKSPACE (ws given
 * but smaller than kvs_topk_workspace(n)).
 */
kvs_status kvs_topk_select(const float* score, int64_t n, int64_t f0_begin, int64_t f0_end,
                           int64_t f1_begin, int64_t f1_end, int64_t C, uint8_t* keep_mask,
                           int32_t* keep_idx, int64_t* n_kept, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * Top-k and slot-map redirect in one launch -- IntentKV Sec. 3.1, Eq. (1),
 * and the layout layer's slot map S_r (abstract; Sec. 1): the selection of
 * kvs_topk_select, bit for bit, whose emit also writes
 *   slot_out[j] = keep_mask[j] ? slot_in[j] : dead_slot
 * as kvs_slotmap_redirect would from the mask.  One eviction step of the
 * rule mode is then this call after kvs_rule_score.  Above 32768 scores
 * (with a workspace) the selection's own emit writes the slot map; a
 * one-workgroup selection is followed by the redirect kernel instead.
 *   slot_in, slot_out  [n] int64, device (may be the same array).
 * Other arguments, workspace and errors as kvs_topk_select (KVS_ERR_ARG also
 * for a null slot array when n > 0).
 */
kvs_status kvs_topk_select_redirect(const float* score, int64_t n, int64_t f0_begin, int64_t f0_end,
                                    int64_t f1_begin, int64_t f1_end, int64_t C, uint8_t* keep_mask,
                                    int32_t* keep_idx, int64_t* n_kept, const int64_t* slot_in,
                                    int64_t dead_slot, int64_t* slot_out, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * Budgeted top-k that allocates nothing -- for callers that cannot allocate:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The same selection as kvs_topk_select, bit for bit, with the
 * same arguments except the workspace: above 32768 scores the multi-workgroup
 * state lives in a static device array of the library (about 66 KB, enough
 * for kvs_topk_noalloc_max() scores), which each device holds from the first
 * call on it until the process ends.  Every call on a device shares that
 * array, so calls that overlap on one device (two streams, two host threads)
 * race and must be ordered by the caller; consecutive calls need nothing, as
 * each rewrites the state it reads.  The first call on a device also resolves
 * the array's address there (no allocation).
 * Errors: as kvs_topk_select, and KVS_ERR_LIMIT when n > kvs_topk_noalloc_max().
 */
int64_t kvs_topk_noalloc_max(void);
kvs_status kvs_topk_select_noalloc(const float* score, int64_t n, int64_t f0_begin, int64_t f0_end,
                                   int64_t f1_begin, int64_t f1_end, int64_t C, uint8_t* keep_mask,
                                   int32_t* keep_idx, int64_t* n_kept, void* stream);

/*
 * Slot-map redirect -- IntentKV layout layer (abstract; Sec. 1 contributions;
 * Sec. 3.1 slot map S_r in Z^N): a dropped position is routed to the sentinel
 * dead slot; kept positions keep their slot, K/V rows and RoPE phase.
 *   slot_out[j] = keep_mask[j] ? slot_in[j] : dead_slot
 *   slot_in, slot_out [N] int64 (may alias); keep_mask [N] uint8.
 * Errors: KVS_ERR_ARG.
 */
kvs_status kvs_slotmap_redirect(const int64_t* slot_in, const uint8_t* keep_mask, int64_t N,
                                int64_t dead_slot, int64_t* slot_out, void* stream);

/*
 * Mean-K index build -- KVMEM, section "Design and trade-offs ... Mean-K":
 * one mean of position-free K per block of `block` tokens, per layer and KV
 * head.  index[l,g,b,:] = bf16( (1/n_b) sum_{i in block b} k~[l,g,i,:] ),
 * summed in float32 from -0 (so a block of -0 keys averages to -0), rounded
 * to nearest-even; a partial last block averages its n_b < block tokens.
 *   K        [L, H_kv, N, D] bf16.  k_is_rope = 0: K is raw (pre-RoPE) and k~ = K.
 *            k_is_rope = 1: K carries RoPE at positions pos0 + i (rotate-half
 *            pairs (i, i+D/2), omega_i = theta^(-2i/D)) and k~ is K rotated
 *            back; raw_k_out (nullable, [L,H_kv,N,D] bf16) then receives k~.
 *   index    [L, H_kv, ceil(N/block), D] bf16 output.
 * Errors: KVS_ERR_ARG (null, pos0 < 0, theta not finite/positive),
 * KVS_ERR_UNSUPPORTED (block != 32, D not 64/128), KVS_ERR_SHAPE (also, in
 * de-RoPE mode with raw_k_out, ceil(N/32) * ceil(L*H_kv / 16) >= 2^24: the
 * launch's grid limit).
 */
kvs_status kvs_meank_build(const void* K, int32_t L, int32_t H_kv, int32_t D, int64_t N,
                           int32_t block, int32_t k_is_rope, int64_t pos0, double theta,
                           void* raw_k_out, void* index, void* stream);

/*
 * Incremental Mean-K append with de-RoPE stage-out -- KVMEM, section
 * "Engineering and cost ...": proactive stage-out writes the raw-K copy (the
 * reconstruction authority) while chunked prefill runs, and the index of the
 * Mean-K section is the per-block mean of that position-free K.
 * Token t of the workspace sits at position pos0 + t.  The chunk holds the
 * post-RoPE keys of tokens t0 .. t0+n_new-1.  For every layer and KV head:
 *   raw_stage[l,g,t,:] = bf16(RoPE(-(pos0 + t)) k_chunk[l,g,t-t0,:])   (t0 <= t < t0+n_new)
 *   index[l,g,b,:] = mean of raw_stage[l,g,32b .. min(32b+32, t0+n_new)-1,:]
 *     for every block b with 32b < t0+n_new and 32b+32 > t0 (the blocks the
 *     chunk touches; a partial last block averages over the tokens it has and
 *     is redone by the next append).
 * After any sequence of appends, the index equals kvs_meank_build run in raw
 * mode on raw_stage[:, :, 0:t0+n_new] bit for bit.
 *   k_chunk    [L, H_kv, n_new, D] bf16, device.
 *   raw_stage  [L, H_kv, cap, D] bf16, device: rows [32*floor(t0/32), t0) are
 *              read (they must hold earlier appends), rows [t0, t0+n_new) written.
 *   index      [L, H_kv, ceil(cap/32), D] bf16, device: touched blocks written.
 *   theta      RoPE base (omega_i = theta^(-2i/D), rotate-half pairing).
 * n_new == 0 is a no-op.  Errors: KVS_ERR_ARG (null, negative, theta not
 * finite and positive), KVS_ERR_SHAPE (t0 + n_new > cap, overflow),
 * KVS_ERR_UNSUPPORTED (D not 64/128).
 */
kvs_status kvs_meank_append(const void* k_chunk, int32_t L, int32_t H_kv, int32_t D, int64_t t0,
                            int64_t n_new, int64_t pos0, double theta, void* raw_stage,
                            int64_t cap, void* index, void* stream);

/* Workspace bytes kvs_meank_score needs. */
size_t kvs_meank_score_workspace(int32_t L, int32_t H_q, int32_t H_kv, int64_t Mq, int64_t nB);

/*
 * Block relevance R_b -- KVMEM, section "Design and trade-offs ... Mean-K":
 * per layer l, query head h and query token m, a softmax over the candidate
 * blocks C of q[l,h,m] . kbar[l,h/G,b] / sqrt(D); summed over m and averaged
 * over the L*H_q (layer, head) pairs.  C = [n_sink, nB - n_recent).
 *   Q        [L, H_q, Mq, D] bf16 position-free query vectors.
 *   index    [L, H_kv, nB, D] bf16 Mean-K index.
 *   R        [nB] float32 output; 0 on sink and recent blocks; sum over C = Mq.
 *   ws       device workspace of >= kvs_meank_score_workspace() bytes.
 * Errors: KVS_ERR_ARG, KVS_ERR_SHAPE (also nB or G*Mq above 2^23 - 128),
 * KVS_ERR_UNSUPPORTED (D not 64/128), KVS_ERR_WORKSPACE.
 */
kvs_status kvs_meank_score(const void* Q, const void* index, int32_t L, int32_t H_q,
                           int32_t H_kv, int32_t D, int64_t Mq, int64_t nB, int64_t n_sink,
                           int64_t n_recent, float* R, void* ws, size_t ws_bytes, void* stream);

/*
 * Re-RoPE scatter into the execution view -- KVMEM, section "Engineering and
 * cost ...": raw K is the reconstruction authority and RoPE is re-applied at
 * the block's new compact position; V carries no position and is copied.
 * For r < n_sel, layer l, KV head g, offset t < block:
 *   k_pool[l,g, block*page_table[r] + t, :] = RoPE(pos_base + block*r + t) k_src[l,g, block*src_block[r] + t, :]
 *   v_pool[l,g, block*page_table[r] + t, :] = v_src[l,g, block*src_block[r] + t, :]
 * RoPE: rotate-half pairs (i, i+D/2), omega_i = theta^(-2i/D), angles reduced
 * in float64, rotation in float32, bf16 nearest-even output.
 *   k_src, v_src [L, H_kv, src_tokens, D] bf16 (src_tokens a multiple of block).
 *   src_block    [n_sel] int32 device, block ids into the source.
 *   page_table   [n_sel] int32 device destination pages, or NULL for r -> r.
 *   k_pool, v_pool [L, H_kv, pool_pages*block, D] bf16 outputs; pages not
 *                named keep their contents.  v_src/v_pool may both be NULL.
 *   err_flag     nullable device int32: set to 1 if a src_block or
 *                page_table entry is out of range (that block is skipped).
 * Errors: KVS_ERR_ARG, KVS_ERR_SHAPE (also n_sel >= 2^23, n_sel * ceil(L*H_kv / 16)
 * >= 2^24 or L*H_kv > 65535: the launches' grid limits), KVS_ERR_UNSUPPORTED
 * (block != 32, D not 64/128).
 */
kvs_status kvs_rerope_scatter(const void* k_src, const void* v_src, int64_t src_tokens,
                              const int32_t* src_block, const int32_t* page_table, int64_t n_sel,
                              int32_t L, int32_t H_kv, int32_t D, int32_t block, int64_t pos_base,
                              double theta, void* k_pool, void* v_pool, int64_t pool_pages,
                              int32_t* err_flag, void* stream);

/* Workspace bytes kvs_working_set_update needs for a pool of pool_pages pages. */
size_t kvs_working_set_workspace(int64_t pool_pages);

/*
 * Differential working-set update of the execution view -- KVMEM, section
 * "Engineering and cost: tiered movement, page-table aliasing and
 * position-consistent reconstruction": consecutive steps' working sets
 * overlap, and only blocks the step selects that the GPU page pool no longer
 * holds (W_t minus G_{t-1}) are materialised again; retained, incoming and
 * outgoing blocks are told apart.
 * prev_blocks (G_{t-1}, the blocks the pool holds, with their pages) and
 * new_blocks (W_t) are strictly ascending block ids; a block's compact index
 * r is its rank, so it sits at positions pos_base + 32r .. +31.
 *   retained  keeps its page.  If its rank moved, its K is rebuilt from raw
 *             K (the reconstruction authority) at its new positions, exactly
 *             as kvs_rerope_scatter writes it; V is untouched.  A retained
 *             block whose rank did not move is not touched at all, so pos_base
 *             must be the value the pool was last written with (a caller that
 *             shifts pos_base re-scatters the whole selection instead).
 *   incoming  takes a free page (one no retained block holds; free pages in
 *             ascending order go to incoming blocks in ascending rank) and is
 *             written like kvs_rerope_scatter: raw K rotated to its compact
 *             positions, V copied.
 *   outgoing  releases its page (contents left as they are).
 *   k_src, v_src   [L, H_kv, src_tokens, D] bf16 raw (position-free) K and V;
 *                  v_src and v_pool may both be NULL.
 *   k_pool, v_pool [L, H_kv, pool_pages*32, D] bf16, updated in place.
 *   pages_out      [n_new] int32: the new page table (page of rank r).
 *   old_rank_out   [n_new] int32: rank in G_{t-1}, -1 for incoming blocks.
 *   outgoing_pages_out [n_prev] int32: released pages in G_{t-1} order (first
 *                  counts_out[2] entries).
 *   counts_out     [3] int64: retained, incoming, outgoing.
 *   err_flag       device int32 set to 1 (never cleared) when a block id is out
 *                  of range or not ascending, a retained page is out of range
 *                  or held twice; then pages_out is all -1 and no pool row is
 *                  written.  May be NULL.
 *   ws             device workspace of >= kvs_working_set_workspace() bytes.
 * Errors: KVS_ERR_ARG, KVS_ERR_SHAPE (n_new or n_prev > pool_pages, src_tokens
 * not a multiple of 32, n_new * ceil(L*H_kv / 8) >= 2^24, overflow),
 * KVS_ERR_UNSUPPORTED (block != 32, D not 64/128), KVS_ERR_WORKSPACE.
 */
kvs_status kvs_working_set_update(const void* k_src, const void* v_src, int64_t src_tokens,
                                  const int32_t* prev_blocks, const int32_t* prev_pages,
                                  int64_t n_prev, const int32_t* new_blocks, int64_t n_new,
                                  int32_t L, int32_t H_kv, int32_t D, int32_t block,
                                  int64_t pos_base, double theta, void* k_pool, void* v_pool,
                                  int64_t pool_pages, int32_t* pages_out, int32_t* old_rank_out,
                                  int32_t* outgoing_pages_out, int64_t* counts_out,
                                  int32_t* err_flag, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVS_H_ */
