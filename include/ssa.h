/*
 * ssa.h -- C ABI of the stratified sparse decode attention library (gfx950).
 *
 * One decode step of one attention layer, for every (sequence b, kv head h):
 *   1. score every cached token cheaply from a fixed subset of RoPE frequency
 *      pairs ("FASA: Frequency-aware Sparse Attention", section 3 stage 1
 *      TIP; the group's queries are averaged as in PIVOT's proxy query);
 *   2. read the top-k tokens -- or the top-p prefix, the shortest run of
 *      highest-scoring tokens holding a fraction p of the approximate
 *      attention mass -- deterministically ("Stratified Sparse Attention
 *      speeds up decoding 2.96x at 1M context", section "Where sparse
 *      attention loses quality");
 *   3. Poisson-sample the remaining tail with probability proportional to
 *      exp(approximate score) and 4. weight each sampled token by the inverse
 *      of its inclusion probability (same page, section "How SSA stratifies
 *      the cache"), then attend exactly over the union (FASA section 3 stage 2
 *      FAC), merging split partials through the online-softmax state
 *      (m, l, acc) ("S2O: Early Stopping for Sparse Attention via Online
 *      Permutation", methodology part 3).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every array argument is a DEVICE pointer, owned by the caller, on
 *           the device current at the call.  The library allocates nothing;
 *           its global state is a per-device cache of one occupancy query (a
 *           constant of the device, filled on first use, atomically) and the
 *           per-device static workspace of ssa_decode_static (a device array
 *           of SSA_STATIC_WORKSPACE_BYTES, with its address looked up once).
 *           q, k_cache, k_rest, v_cache, k_new and v_new must be 16-byte
 *           aligned.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = null stream).
 *           Calls enqueue work and return; nothing is synchronised.
 * Errors.   0 on success, a negative SSA_ERR_* code otherwise; no partial
 *           work is enqueued when argument validation fails.  Host-visible
 *           arguments (params, pointers, sizes) are validated; device-resident
 *           values are not: seq_lens are clamped to [0, max_seq_len],
 *           negative topk / sample_budget act as 0, topk above a positive
 *           params.max_topk acts as max_topk, and block_table entries
 *           are clamped to [0, num_blocks) (a wrong entry reads a wrong block,
 *           never out of bounds).
 * Determinism. No floating-point atomics are used: identical inputs and
 *           seeds give bitwise identical outputs, and calls are reentrant.
 *
 * Query positions.  A step carries T >= 1 query positions per sequence
 *   (params.num_queries; multi-token decode).  seq_lens[b] = P_b is the cache
 *   length with the T new tokens' keys already in it: query t sits at
 *   position P_b - T + t and attends to tokens [0, P_b - T + t].  Queries are
 *   grouped g = params.query_group consecutive at a time (the last group may
 *   be smaller); a group is scored once with its proxy query, the mean of its
 *   members' queries ("PIVOT slashes sparse-attention indexer cost", "The two
 *   observations behind PIVOT"), and its one selection serves every member,
 *   each restricted to its own span.  NG = ceil(T / g) groups per sequence.
 *   Selection units are u = (b * NG + group) * Hkv + h (with params.refine,
 *   every member's own: see "Refine mode").  T = g = 1 is plain one-token
 *   decode.
 *
 * Layouts (row-major, innermost last)
 *   q            [B, T, Hq, d]                   bf16 (post-RoPE queries)
 *   k_cache      [num_blocks, Hkv, 16, d]        bf16 (post-RoPE keys, interleaved pairs)
 *   v_cache      [num_blocks, Hkv, 16, d]        bf16
 *   block_table  [B, max_blocks_per_seq]         int32: token j of sequence b is row
 *                                                j % 16 of block block_table[b][j / 16]
 *   seq_lens, topk, sample_budget [B]            int32
 *   top_p        [B]                             f32, optional (NULL = top-k only)
 *   seed         [B]                             uint64 (one Philox key per sequence)
 *   out          [B, T, Hq, d]                   f32 or bf16 (params.out_dtype)
 *
 * Split keys (params.key_layout = SSA_KEYS_SPLIT; "FASA: Frequency-aware
 * Sparse Attention", section 3, variants: FASA-M keeps the dominant key
 * components on the GPU and moves the rest of the key and the whole value
 * cache to host memory).  A key row is stored as two rows of the same row
 * number: the scored dims and the others.
 *   k_cache (k_dom) [num_blocks, Hkv, 16, 2 * pair_count]      dims [2 pb, 2 (pb + pc))
 *   k_rest          [num_blocks, Hkv, 16, d - 2 * pair_count]  dims [0, 2 pb) then
 *                                                              [2 (pb + pc), d)
 *   The indexer reads k_dom only; attention reads the selected rows of
 *   k_dom, k_rest and v_cache.  k_rest and v_cache may be pinned host
 *   memory that the device can address (hipHostMalloc; pass the address
 *   that hipHostGetDevicePointer returns): then the GPU holds
 *   2 * pair_count of the 4 * d key and value elements per token.
 *
 * Selection layout (ssa_select output, ssa_attend input).  A sequence's
 * positions are cut into chunks of SSA_CHUNK_TOKENS; NC = ssa_num_chunks().
 *   sel_idx   [B, NG, Hkv, NC * SSA_CHUNK_TOKENS]  int32 token positions
 *   sel_logw  [B, NG, Hkv, NC * SSA_CHUNK_TOKENS]  f32   logit bias -log(pi_j): 0 on the
 *                                                     deterministic set, >= 0 on samples
 *   sel_count [B, NG, Hkv, NC, 2]                  int32 (n_det, n_sampled) of each chunk
 *   Segment c of a unit starts at c * SSA_CHUNK_TOKENS and holds the chunk's
 *   deterministic tokens (ascending) followed by its sampled tokens
 *   (ascending).  Chunks at or past L_b have count (0, 0).
 */
#ifndef SSA_H_
#define SSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SSA_OK 0
#define SSA_ERR_INVALID (-1)   /* bad params, null or misaligned pointer, bad size */
#define SSA_ERR_WORKSPACE (-2) /* workspace smaller than ssa_workspace_bytes()     */
#define SSA_ERR_HIP (-3)       /* a HIP call or kernel launch failed               */
#define SSA_ERR_STATIC_LIMIT (-4) /* the step needs more workspace than             */
                                  /* SSA_STATIC_WORKSPACE_BYTES (ssa_decode_static) */

/* Output element types. */
#define SSA_F32 0
#define SSA_BF16 1

/* Key layouts. */
#define SSA_KEYS_WHOLE 0 /* k_cache holds whole key rows                           */
#define SSA_KEYS_SPLIT 1 /* k_cache holds the scored dims, k_rest the others       */

#define SSA_BLOCK_TOKENS 16    /* tokens per KV-cache block (the only size supported) */
#define SSA_CHUNK_TOKENS 4096  /* selection / split granularity                      */
#define SSA_MAX_SEQ_LEN (1 << 24) /* 4096 chunks of 4096 tokens */

/* Stage indices for ssa_decode_timed(). */
#define SSA_STAGE_INIT 0     /* clear histograms and maxima                        */
#define SSA_STAGE_INDEX 1    /* approximate scores + first-digit histogram + max   */
#define SSA_STAGE_FILTER 2   /* (top-p mass histogram,) first-digit threshold,      */
                             /* candidates, tail weight sums                        */
#define SSA_STAGE_RESOLVE 3  /* exact top-k threshold, tie quota, tail normaliser  */
#define SSA_STAGE_SAMPLE 4   /* deterministic set + Poisson sample, per chunk      */
                             /* (without early stopping or refine, taken by the    */
                             /* attention kernel: no kernel here)                 */
#define SSA_STAGE_ATTEND 5   /* gather attention over the selection, split-K       */
#define SSA_STAGE_MERGE 6    /* merge of the split partials                        */
#define SSA_NUM_STAGES 7

typedef struct ssa_params {
  int32_t batch;              /* B >= 1                                                  */
  int32_t num_q_heads;        /* Hq, a multiple of Hkv, Hq / Hkv <= 16                   */
  int32_t num_kv_heads;       /* Hkv >= 1                                                */
  int32_t head_dim;           /* d: 64 or 128                                            */
  int32_t block_size;         /* must be SSA_BLOCK_TOKENS                                */
  int32_t max_blocks_per_seq; /* columns of block_table                                  */
  int32_t num_blocks;         /* rows of k_cache / v_cache                               */
  int32_t max_seq_len;        /* upper bound of seq_lens; <= max_blocks_per_seq * 16     */
  int32_t pair_begin;         /* first scored RoPE pair (pairs are dims (2p, 2p+1));      */
                              /*   a multiple of 4                                        */
  int32_t pair_count;         /* 4, 8, 16, 32 or 64 pairs; pair_begin + pair_count <= d/2 */
  int32_t num_splits;         /* split-K slices per query position and kv head;          */
                              /*   0 = one per chunk                                      */
  int32_t out_dtype;          /* SSA_F32 or SSA_BF16                                     */
  float softmax_scale;        /* > 0; 0 selects 1 / sqrt(d)                              */
  int32_t num_queries;        /* T >= 1 query positions per sequence                     */
  int32_t query_group;        /* g >= 1 consecutive queries sharing one selection        */
  float early_stop;           /* tau of the early-stopping rule below; <= 0 or NaN = off */
  int32_t key_layout;         /* SSA_KEYS_WHOLE or SSA_KEYS_SPLIT                         */
  int32_t max_topk;           /* >= 0: an upper bound of topk[b] (larger device values    */
                              /*   act as it); 0 = max_seq_len.  Early stopping needs     */
                              /*   it (or max_seq_len) <= SSA_STOP_MAX_STRATUM            */
  int32_t refine;             /* >= 0: 0 = query groups reuse the group's selection;     */
                              /*   r >= 1 = every member refines a candidate list of      */
                              /*   r * topk tokens (see "Refine mode" below)              */
} ssa_params;

/* Largest deterministic stratum the early-stopping kernels order (tokens). */
#define SSA_STOP_MAX_STRATUM 16384
/* Largest number of query rows (members x query heads) of one selection unit
 * that early stopping weighs. */
#define SSA_STOP_MAX_ROWS 16

/* Bytes of device workspace that ssa_decode / ssa_score / ssa_select /
 * ssa_attend need for these params (0 if params are invalid).  The workspace
 * holds no state between calls. */
size_t ssa_workspace_bytes(const ssa_params* p);

/* ceil(max_seq_len / SSA_CHUNK_TOKENS) (0 if params are invalid). */
int32_t ssa_num_chunks(const ssa_params* p);

/* The whole decode step: scores, selection, sampling, attention, merge.
 *
 * Deterministic stratum.  Tokens are ordered by score (float32, larger first;
 * ties to the lower position).  The stratum is the first k tokens of that
 * order, k = min(topk[b], L_b) -- further capped, when top_p is non-NULL, by
 * n_p, the length of the shortest prefix whose approximate mass reaches
 * top_p[b].  Mass is counted exactly in integer units: token j holds
 * floor(w_j * 2^38) units, w_j = exp(s_j - M) with the library's specified
 * float32 exp (M the sequence's maximum score, so the top token holds 2^38),
 * and the prefix must reach ceil(p * Q) units of the sequence's total Q
 * (0 units -> n_p = 0).  top_p[b] is clamped to [0, 1]; NaN counts as 0.
 * To use top-p alone pass topk[b] >= L_b.
 *
 * Early stopping ("S2O: Early Stopping for Sparse Attention via Online
 * Permutation", methodology parts 2 and 3).  With params.early_stop = tau > 0
 * the stratum, in its order, is visited in blocks of 64 tokens while the
 * online-softmax state of every query row of the unit (each query head of
 * each member of the query group; a row sees only tokens inside its member's
 * span) takes in the block's exact attention mass; the visit stops after the
 * first block at which, for every row, the block's gain in the row's softmax
 * denominator l is 0 or below tau times the row's l so far (tau above 1 acts
 * as 1).  The rest of the stratum is skipped: neither read nor sampled; the
 * tail sample is unchanged.  The decision is exact and reproducible: the
 * logit is fl32(scale * dot), the dot of bf16 values summed in float32 (each
 * 8-dim slice in dim order, then the slices pairwise), and gains are counted
 * in the integer units above, floor(2^38 exp(l - M_row)) with the specified
 * exp and M_row the row's largest logit over the stratum.  Requires the
 * stratum bound (params.max_topk, or max_seq_len when it is 0) to be at most
 * SSA_STOP_MAX_STRATUM and the unit's query rows (min(query_group,
 * num_queries) x Hq / Hkv) at most SSA_STOP_MAX_ROWS; otherwise every entry
 * point returns SSA_ERR_INVALID.  Cost: ordering the stratum and weighing it
 * takes seven short kernels, about 50 us per step for a 1M-token layer of 8
 * kv heads with a 10486-token stratum, and the step then runs the sample
 * stage as its own kernel (measured: 230 us -> 292 us per step at tau =
 * 0.01, which cuts the stratum by 57%), far more than the attention it saves
 * at 50x sparsity (about 2 us); it pays only where attention over the stratum
 * dominates the step.
 *
 * Refine mode ("PIVOT slashes sparse-attention indexer cost", "The two
 * observations behind PIVOT" and "Two operating modes": the proxy's
 * candidate list is refined for each member).  With params.refine = r >= 1
 * the group's selection runs with a stratum of r * topk tokens, the
 * candidate list C; each member t (query position) then scores C's tokens
 * inside its span with its own query -- per head the float32 dot over the
 * scored dims (8-dim slices in dim order, then the slices pairwise), the
 * heads summed in head order, times fl32(fl32(scale) / G) -- and keeps the
 * first k_t = min(topk, |C inside its span|) of them in the order (own score
 * descending, position ascending); it is dense when k_t + m reaches its span.
 * Its tail is the group's span minus its stratum, sampled with the proxy's
 * weights exp(s_j - M), the group's Philox stream and its own normaliser
 * W_t (the sum of those weights over its tail).  Every member then has its
 * own selection: ssa_select writes, ssa_attend reads and w_in / norm_out
 * hold one selection unit per (b, t, h), u = (b * T + t) * Hkv + h, in the
 * layout below with NG = T.  Not combined with top_p or early stopping
 * (SSA_ERR_INVALID); the group's staged query slices, min(query_group,
 * num_queries) * Hq / Hkv * 2 * pair_count floats, must be at most 8192.
 *
 * Tail.  sample_budget[b] (m) is the expected number of tail samples.  If
 * k + m >= L_b every token is read with weight 1 (dense attention).
 * Sampling for (b, h, token j) uses Philox4x32-10 keyed by seed[b] with
 * counter (j >> 2, h, b, 0), word j & 3 (Salmon et al., SC'11). */
int ssa_decode(const ssa_params* p, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const int32_t* seq_lens, const int32_t* topk,
               const float* top_p, const int32_t* sample_budget, const uint64_t* seed, void* out,
               void* workspace, size_t workspace_bytes, void* stream);

/* Size of the device array that ssa_decode_static uses as its workspace:
 * 128 MiB, held by every device the library runs on until the process ends.
 * It covers, for example, a 128K-token layer of batch 4 with 8 kv heads. */
#define SSA_STATIC_WORKSPACE_BYTES ((size_t)128 << 20)

/* ssa_decode for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step, bitwise the same output, with the workspace taken from a device
 * array of SSA_STATIC_WORKSPACE_BYTES that the library holds per device
 * (its address is looked up once per device, on the first call with that
 * device current).  Allocates nothing.  Returns SSA_ERR_STATIC_LIMIT, before
 * any launch, when ssa_workspace_bytes(p) exceeds that size.  Every call on a
 * device shares that device's array, so calls that overlap on one device
 * (other streams or threads) race; calls in one stream are ordered. */
int ssa_decode_static(const ssa_params* p, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* topk, const float* top_p, const int32_t* sample_budget,
                      const uint64_t* seed, void* out, void* stream);

/* ssa_decode, recording hipEvent_t events[2*s] before and events[2*s+1] after
 * the kernel(s) of stage s (SSA_STAGE_*); NULL entries are skipped, and a
 * NULL array records nothing.  Same results as ssa_decode.  ssa_decode and
 * ssa_decode_timed take whole keys (params.key_layout = SSA_KEYS_WHOLE). */
int ssa_decode_timed(const ssa_params* p, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                     const int32_t* topk, const float* top_p, const int32_t* sample_budget,
                     const uint64_t* seed, void* out, void* workspace, size_t workspace_bytes,
                     void* stream, void* const* events);

/* ssa_decode over split keys (params.key_layout = SSA_KEYS_SPLIT): k_dom
 * holds the scored dims and k_rest the others (layouts above; k_rest may be
 * NULL only when 2 * pair_count = d).  events as for ssa_decode_timed (may be
 * NULL).  The same arithmetic in the same order as ssa_decode: the output is
 * bitwise that of ssa_decode on the whole keys the two arrays hold. */
int ssa_decode_split(const ssa_params* p, const void* q, const void* k_dom, const void* k_rest,
                     const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                     const int32_t* topk, const float* top_p, const int32_t* sample_budget,
                     const uint64_t* seed, void* out, void* workspace, size_t workspace_bytes,
                     void* stream, void* const* events);

/* Stage 1 alone ("FASA: Frequency-aware Sparse Attention", section 3 stage 1
 * TIP: a token's online score sums the contributions of a fixed subset of
 * RoPE frequency chunks; the query group is averaged into one proxy query as
 * in "PIVOT slashes sparse-attention indexer cost", "The two observations
 * behind PIVOT"): approximate scores, scores[u * max_seq_len + j] (f32) of
 * selection unit u = (b * NG + group) * Hkv + h, for j below the group's span
 * (its last member's causal length); later entries are left untouched.
 *   s_j = (1/(n G)) sum over the group's n members and G heads of
 *         scale * sum_{p in pairs} (q[2p] k_j[2p] + q[2p+1] k_j[2p+1]).
 * k_cache holds whole keys or, with SSA_KEYS_SPLIT, the scored dims only.
 * Errors as for ssa_decode. */
int ssa_score(const ssa_params* p, const void* q, const void* k_cache,
              const int32_t* block_table, const int32_t* seq_lens, float* scores,
              void* workspace, size_t workspace_bytes, void* stream);

/* Stages 2-4 alone ("Stratified Sparse Attention speeds up decoding 2.96x
 * at 1M context", sections "Where sparse attention loses quality" and "How
 * SSA stratifies the cache": the top-k or top-p stratum read
 * deterministically, the tail Poisson-sampled with probability proportional
 * to exp(score) and weighted by the inverse inclusion probability), from a
 * caller-provided score array laid out as ssa_score writes it (one row per
 * selection unit, valid over the unit's span); topk, top_p (may be NULL) and
 * sample_budget as for ssa_decode.  Sampling for (b, group, h, token j) uses
 * counter (j >> 2, h, b, group).  If w_in is non-NULL, w_in[u] replaces the
 * computed tail normaliser W of unit u.  Writes the selection (layout above)
 * and norm_out [B, NG, Hkv, 2] = (M, W): the maximum score and the normaliser
 * actually used.  q, k_cache, k_rest and block_table are read only by early
 * stopping (params.early_stop > 0), which weighs the stratum by exact
 * attention (k_rest as for ssa_decode_split with SSA_KEYS_SPLIT, else NULL);
 * they may be NULL when it is off.  Errors as for ssa_decode; the score
 * array is not validated (non-finite scores select arbitrarily but stay in
 * bounds). */
int ssa_select(const ssa_params* p, const float* scores, const int32_t* seq_lens,
               const int32_t* topk, const float* top_p, const int32_t* sample_budget,
               const uint64_t* seed, const float* w_in, const void* q, const void* k_cache,
               const void* k_rest, const int32_t* block_table, int32_t* sel_idx, float* sel_logw,
               int32_t* sel_count, float* norm_out, void* workspace, size_t workspace_bytes,
               void* stream);

/* Stages 5-6 alone ("FASA: Frequency-aware Sparse Attention", section 3
 * stage 2 FAC: full-precision attention on the selected tokens at their
 * original positions; the inverse-inclusion-probability weights of "How SSA
 * stratifies the cache" enter as logit biases; split partial states
 * (m, l, acc) are merged as in "S2O: Early Stopping for Sparse Attention via
 * Online Permutation", methodology part 3): attention over a caller-provided
 * selection (one per selection unit), for every query position t and head g
 * of the unit's group:
 *   out_g = sum_A e^{l_gj + logw_j} v_j / sum_A e^{l_gj + logw_j},
 *   l_gj = scale * q_g . k_j over the full head dimension, A = the unit's
 *   selected positions below the query's span (later ones are ignored).
 * Counts are clamped to a chunk's segment and positions to the span, so a
 * malformed selection reads wrong rows, never out of bounds.  Errors as for
 * ssa_decode. */
int ssa_attend(const ssa_params* p, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const int32_t* seq_lens, const int32_t* sel_idx,
               const float* sel_logw, const int32_t* sel_count, void* out, void* workspace,
               size_t workspace_bytes, void* stream);

/* ssa_attend over split keys (params.key_layout = SSA_KEYS_SPLIT); k_rest
 * as for ssa_decode_split.  Bitwise the output of ssa_attend on the whole
 * keys. */
int ssa_attend_split(const ssa_params* p, const void* q, const void* k_dom, const void* k_rest,
                     const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                     const int32_t* sel_idx, const float* sel_logw, const int32_t* sel_count,
                     void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Append num_tokens = T new tokens per sequence to the cache: token t of
 * sequence b goes to position seq_lens[b] - T + t (seq_lens counting the new
 * tokens, as for ssa_decode), row (pos % 16) of block block_table[b][pos / 16];
 * positions below 0 are skipped.  k_new, v_new: [B, T, Hkv, d] bf16
 * (post-RoPE keys).  With SSA_KEYS_WHOLE k_cache receives whole key rows and
 * k_rest must be NULL; with SSA_KEYS_SPLIT k_cache receives the scored dims
 * and k_rest the others (NULL only when 2 * pair_count = d).  v_cache
 * receives the values.  Caches may be pinned host memory as above.  Rows
 * that two new tokens of one call share receive one of them.  Needs no
 * workspace; B * T may be as large as the cache (bulk fill, e.g. after a
 * prefill), below 2^31.  Requires Hkv * d <= 8192. */
int ssa_append_kv(const ssa_params* p, int32_t num_tokens, const void* k_new, const void* v_new,
                  const int32_t* block_table, const int32_t* seq_lens, void* k_cache,
                  void* k_rest, void* v_cache, void* stream);

/* The device address of pinned host memory (hipHostMalloc), for passing
 * offloaded caches (k_rest, v_cache) to the calls above: *dev_ptr receives
 * the address kernels use for host_ptr.  SSA_ERR_INVALID if host_ptr is not
 * pinned, device-mapped memory (the caller must not pass it then). */
int ssa_host_device_address(const void* host_ptr, void** dev_ptr);

/* Test hook: words[i] = the Philox word of (seed, b, h, group, token j0 + i), i < n. */
int ssa_debug_philox(uint64_t seed, int32_t b, int32_t h, int32_t group, int32_t j0, int32_t n,
                     uint32_t* words, void* stream);

/* Test hook: y[i] = the library's specified float32 exp of x[i], i < n. */
int ssa_debug_sexp(const float* x, float* y, int32_t n, void* stream);

/* Test hook: y[i] = the chunk filter's first-pass tail weight e^x[i] (the
 * hardware exp2 with an extended-precision argument; 0 below -87), i < n.
 * It enters only the library's own tail sum W and the necessary inclusion
 * test, never an exact decision. */
int ssa_debug_tail_exp(const float* x, float* y, int32_t n, void* stream);

/* Measurement aids, not steps of the decode: the HBM read rate this device
 * delivers for the access patterns of the step's two bandwidth-bound
 * kernels, so that their achieved rates can be set beside what the memory
 * gives for the same pattern (the published peak is not reachable by any
 * access pattern).  Each folds every 32-bit word it reads by XOR into the
 * sink, an array of SSA_MEASURE_SINK_WORDS words (integer atomics spread over
 * the array; the result does not depend on the order of the work): clear the
 * sink first, and the XOR of its words afterwards is the XOR of the data.
 *   ssa_measure_stream: bytes (a positive multiple of 16) read contiguously
 *     from src, the indexer's pattern (a long stream).
 *   ssa_measure_gather: n rows of row_bytes (a power of two, 16 to 1024) at
 *     src + rows[i] * row_bytes, rows[i] clamped to [0, num_rows) -- src
 *     must hold num_rows such rows -- the attention's pattern (selected K
 *     and V rows, scattered over the cache).
 * src must be 16-byte aligned.  SSA_ERR_INVALID on a null pointer or a size
 * out of range; n = 0 enqueues nothing. */
#define SSA_MEASURE_SINK_WORDS 4096
int ssa_measure_stream(const void* src, size_t bytes, uint32_t* sink, void* stream);
int ssa_measure_gather(const void* src, size_t row_bytes, int64_t num_rows, const int32_t* rows,
                       int64_t n, uint32_t* sink, void* stream);

/* Static description of a status code. */
const char* ssa_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* SSA_H_ */
