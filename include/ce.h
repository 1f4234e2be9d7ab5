/*
 * ce.h - C ABI of the centroid-masked sparse LM head for MI355X (gfx950).
 *
 * The operation is the one of Gemma4MTPMaskedEmbedder in the vLLM compare view
 * "[Spec Decode] Add Gemma4 MTP speculative decoding with centroids masking"
 * (diff of gemma4_mtp.py):
 *   _select_and_score  project each hidden row onto Nc centroid vectors, keep
 *                      the K best centroids, gather the embeddings of the
 *                      tokens those centroids own and dot them with the row;
 *   forward            a full-vocabulary logit row: those scores at the
 *                      candidate token ids, the fill value everywhere else;
 *   get_top_tokens     the token id of the largest candidate score.
 *
 * Numerics (fixed where the page leaves them open):
 *   - Every dot product is the canonical key: elements widened exactly to
 *     float64, summed in hidden-dimension order from +0.0 with one rounding
 *     per step (s = fma(x_k, w_k, s)), then rounded to fp32 nearest-even and
 *     -0 turned into +0.  All scores and logits returned are these values.
 *   - Top-K ties go to the lowest centroid id; argmax ties to the lowest token
 *     id.  Top-K ids are returned as an ascending set.
 *   - The fill value of the full-vocabulary row is -inf (fp32 0xFF800000).
 *   - Inputs must be finite: with a NaN or an infinity in h, the centroids
 *     or the embeddings (an infinity can make a NaN product), scores, ids
 *     and tokens are unspecified.  No call checks for this or fails on it.
 *
 * Layout: the embedding table is in the ordered layout: row j holds the
 * embedding of token token_of_slot[j], and cluster c owns the contiguous slots
 * [cluster_offsets[c], cluster_offsets[c+1]).  With equal clusters (offsets
 * NULL) cluster c owns slots [c*V/Nc, (c+1)*V/Nc), which is the page's
 * token_ordering.view(num_centroids, vocab_size_per_centroid).
 *
 * Memory and streams: the library never allocates device memory.  The caller
 * passes a persistent buffer at prepare time and a workspace on every call,
 * sized by ce_head_persistent_bytes / ce_workspace_bytes.  Every compute call
 * is enqueued on the caller's stream, never synchronises, reads no device
 * memory on the host and may be captured into a HIP graph.  Calls that share
 * one workspace must be ordered on one stream.  A head handle is read-only
 * after ce_head_prepare, so calls on several streams with separate
 * workspaces may run concurrently.
 *
 * Errors: every entry point returns a ce_status; nothing is thrown across
 * the ABI.  ce_last_error() gives a thread-local message for the last failure
 * of the calling thread.  Argument checks happen before any device work; on a
 * check failure nothing is enqueued and no output is written.
 */
#ifndef CE_H_
#define CE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ce_status {
  CE_SUCCESS = 0,
  CE_ERR_NULL_POINTER = 1,     /* a required pointer is NULL */
  CE_ERR_BAD_SHAPE = 2,        /* a size is out of range (see each call) */
  CE_ERR_BAD_DTYPE = 3,        /* element type is not CE_F32 or CE_BF16 */
  CE_ERR_MISALIGNED = 4,       /* a device pointer is not 16-byte aligned */
  CE_ERR_BAD_LAYOUT = 5,       /* token_of_slot not a permutation, or bad offsets */
  CE_ERR_WORKSPACE_TOO_SMALL = 6,
  CE_ERR_NOT_PREPARED = 7,     /* compute call before ce_head_prepare */
  CE_ERR_HIP = 8,              /* the HIP runtime reported an error */
  CE_ERR_UNSUPPORTED = 9       /* valid request this library does not serve */
} ce_status;

typedef enum ce_dtype {
  CE_F32 = 0,   /* IEEE binary32 */
  CE_BF16 = 1   /* bfloat16 (upper half of a binary32) */
} ce_dtype;

/* Storage of the embedding slabs the gather reads (ce_head_desc.slab_format).
 *   CE_SLAB_NATIVE    the head's dtype (default; zero-initialised descs)
 *   CE_SLAB_FP8_E4M3  bf16 heads only: each ordered row j stored as OCP
 *                     8-bit E4M3 codes q_jk = E4M3(fl64(E[j,k] / s_j)) (round
 *                     to nearest even, saturating at 448) with the float32
 *                     scale s_j = fl32(max_k |E[j,k]| / 448) (1 for a zero
 *                     row), packed at prepare time.  Candidate logits become
 *                     fl32(fl64(acc * s_j)) with acc the canonical float64
 *                     chain over the decoded codes; centroid scores and top-K
 *                     are unchanged (the centroids stay bf16).  Half the
 *                     gathered bytes; the error against the bf16 head is at
 *                     most sum_k |h_k| (2^-4 |E[j,k]| + 2^-10 s_j) plus the
 *                     final rounding.  The pages do not quantise; this is a
 *                     reduced-precision option with numerics of its own. */
typedef enum ce_slab {
  CE_SLAB_NATIVE = 0,
  CE_SLAB_FP8_E4M3 = 1
} ce_slab;

/* Matrix-core use of the fused calls (ce_head_desc.projection): the
 * centroid projection, and the sparse dot of ce_top_tokens.  The results are
 * the same either way; only the time differs.
 *   CE_PROJ_AUTO   fp32 heads: CE_PROJ_EXACT.  bf16 heads: the projection
 *                  per pass of rows by matrix cores when B*Nc*d >= 2^26
 *                  multiply-adds, where it is the faster; ce_top_tokens'
 *                  dot by matrix cores for d >= 512 or clusters of unequal
 *                  tile counts (above 4 rows on equal ones), else exact
 *   CE_PROJ_EXACT  every score and logit is the canonical key (a float64
 *                  chain) before it is compared
 *   CE_PROJ_MFMA   bf16 heads only, everywhere it applies: the projection is
 *                  the matrix cores' fp32 sums, each within a bound E of its
 *                  canonical key (from |h| and the largest centroid norm),
 *                  with a top-K that recomputes canonical keys wherever E
 *                  leaves the K-th place open; ce_top_tokens' candidate
 *                  logits likewise (E from |h| and each slot's |e|), with a
 *                  finalize that recomputes canonical keys wherever the
 *                  bounds leave the argmax open.  The selected centroids and
 *                  tokens are exactly those of CE_PROJ_EXACT.  Batches of at
 *                  most 4 rows on clusters of equal tile counts keep the
 *                  float64 dot.
 * ce_score_centroids (whose output is the keys) and ce_draft_step always
 * compute canonical scores; ce_masked_logits and ce_top_m always compute
 * canonical logits. */
typedef enum ce_projection {
  CE_PROJ_AUTO = 0,
  CE_PROJ_EXACT = 1,
  CE_PROJ_MFMA = 2
} ce_projection;

typedef enum ce_op {
  CE_OP_SCORE = 0,          /* ce_score_centroids */
  CE_OP_TOPK = 1,           /* ce_topk */
  CE_OP_TOP_TOKENS = 2,     /* ce_top_tokens */
  CE_OP_MASKED_LOGITS = 3,  /* ce_masked_logits */
  CE_OP_TOP_M = 4,          /* ce_top_m */
  CE_OP_DRAFT_STEP = 5,     /* ce_draft_step */
  CE_OP_TOP_M_LOG_SOFTMAX = 6  /* ce_top_m_log_softmax */
} ce_op;

typedef struct ce_head* ce_head_t;
typedef struct ce_graph* ce_graph_t;

/* Shape and weights of one head (the constructor arguments of the page's
 * Gemma4MTPMaskedEmbedder: hidden_size, vocab_size, num_centroids,
 * centroid_intermediate_top_k, plus the centroid weight, token_ordering and
 * the lm_head weight that _select_and_score receives).
 *
 *   d        hidden size; a multiple of 64 in [64, 8192]
 *   V        vocabulary size, in [1, 2^31 - 1]
 *   Nc       number of centroids, in [1, 8192] and <= V when offsets is NULL
 *   max_B    largest batch any call will pass, >= 1
 *   max_K    largest K any call will pass, in [1, Nc]
 *   dtype    element type of h, centroids and embeddings (ce_dtype)
 *   centroids       DEVICE [Nc][d] row-major, 16-byte aligned
 *   emb_ordered     DEVICE [V][d] row-major, 16-byte aligned; row j is the
 *                   embedding of token token_of_slot[j]
 *   cluster_offsets HOST [Nc+1] nondecreasing, offsets[0] = 0,
 *                   offsets[Nc] = V; or NULL for equal clusters (V % Nc == 0).
 *                   Empty clusters are allowed.  Copied at create.
 *   token_of_slot   HOST [V], a permutation of 0..V-1.  Copied at create.
 *   slab_format     ce_slab; CE_SLAB_FP8_E4M3 needs dtype CE_BF16.
 *   projection      ce_projection; CE_PROJ_MFMA needs dtype CE_BF16.
 * The two device arrays are read only by ce_head_prepare, which packs them
 * into the persistent buffer; they may be freed or changed afterwards. */
typedef struct ce_head_desc {
  int32_t d;
  int32_t V;
  int32_t Nc;
  int32_t max_B;
  int32_t max_K;
  int32_t dtype;
  const void* centroids;
  const void* emb_ordered;
  const int32_t* cluster_offsets;
  const int32_t* token_of_slot;
  int32_t slab_format;
  int32_t projection;
} ce_head_desc;

/* Validate desc on the host and create a head.  Makes no HIP call.
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_DTYPE, MISALIGNED, BAD_LAYOUT. */
ce_status ce_head_create(const ce_head_desc* desc, ce_head_t* out);

/* Release a head (host memory only; the caller owns every device buffer).
 * NULL is accepted. */
ce_status ce_head_destroy(ce_head_t head);

/* Bytes of the persistent device buffer ce_head_prepare needs. Host only. */
ce_status ce_head_persistent_bytes(ce_head_t head, size_t* bytes);

/* Fill the caller's persistent device buffer (256-byte aligned, at least
 * ce_head_persistent_bytes): the derived tables (offsets, the slot->token
 * map, the list of 64-slot cluster tiles and each tile's slot tokens) and
 * packed copies of the centroids and embeddings (quantised for FP8 slabs,
 * with their row scales) in 64-row tiles whose 16-byte vectors are
 * interleaved across rows, so that the hot kernels stream them with fully
 * coalesced loads (one more copy of the weights in HBM).  Set-up
 * only: copies and packs on `stream` and synchronises it.  The buffer must
 * live as long as the head is used.
 * Errors: NULL_POINTER, MISALIGNED, WORKSPACE_TOO_SMALL, HIP. */
ce_status ce_head_prepare(ce_head_t head, void* persistent, size_t bytes,
                          hipStream_t stream);

/* Workspace bytes one call of `op` with batch B and top-K K needs (the
 * worst case over inputs).  Host only.  CE_OP_SCORE and CE_OP_TOPK need none
 * (0 bytes).
 * Errors: NULL_POINTER, BAD_SHAPE. */
ce_status ce_workspace_bytes(ce_head_t head, int32_t B, int32_t K, int32_t op,
                             size_t* bytes);

/* The centroid projection (the page's self.centroids(hidden_states)):
 *   scores[b][c] = canonical dot(h[b], centroids[c]),  b < B, c < Nc.
 *   h       DEVICE [B][d] of the head's dtype, 16-byte aligned
 *   scores  DEVICE [B][Nc] fp32, written entirely
 * No workspace.  B = 0 is a no-op.  Errors: NOT_PREPARED, NULL_POINTER,
 * BAD_SHAPE (B outside [0, max_B]), MISALIGNED, HIP. */
ce_status ce_score_centroids(ce_head_t head, const void* h, int32_t B,
                             float* scores, hipStream_t stream);

/* Top-K selection (the page's torch.topk over the centroid scores) on a
 * caller-given fp32 array, bit-exact: topk_ids[b] holds, in ascending order,
 * the K centroid ids that rank first under (score descending, id ascending),
 * with -0 equal to +0.
 *   scores    DEVICE [B][Nc] fp32 (no NaN)
 *   topk_ids  DEVICE [B][K] int32
 * No workspace.  B = 0 is a no-op.  Errors: NOT_PREPARED, NULL_POINTER,
 * BAD_SHAPE (B outside [0, max_B], K outside [1, max_K]), HIP. */
ce_status ce_topk(ce_head_t head, const float* scores, int32_t B, int32_t K,
                  int32_t* topk_ids, hipStream_t stream);

/* get_top_tokens: for every row b < B, the token id t with the largest
 * canonical logit among the tokens owned by the row's K selected centroids,
 * ties to the lowest id; -1 when those centroids own no token (possible only
 * with empty clusters).
 *   h                DEVICE [B][d] of the head's dtype, 16-byte aligned
 *   tokens           DEVICE [B] int32
 *   topk_ids_or_null DEVICE [B][K] int32 (the selected centroids, ascending)
 *                    or NULL
 *   ws               DEVICE workspace, 256-byte aligned
 * B = 0 is a no-op.  Rows are independent: row b's outputs do not depend on
 * B or on the other rows.  Errors: as ce_score_centroids, plus BAD_SHAPE for
 * K outside [1, max_K]. */
ce_status ce_top_tokens(ce_head_t head, const void* h, int32_t B, int32_t K,
                        int32_t* tokens, int32_t* topk_ids_or_null, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* ce_top_tokens for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops, harnesses that forbid hipMalloc): the
 * same call and results without the workspace arguments.  Its workspace is a
 * static array of the library, CE_STATIC_SCRATCH_BYTES on each GPU, held
 * until the process ends; the call allocates nothing.  Every call on one GPU
 * shares that GPU's array, so calls that may overlap on one GPU (on several
 * streams, or from several threads without ordering) race and must not be
 * issued; calls ordered on one stream are safe.  The array's content is not
 * needed from one call to the next (every region is written before it is
 * read).  When the matrix-core argmax's records (16 bytes per row and tile,
 * part of ce_workspace_bytes(head, B, K, CE_OP_TOP_TOKENS)) would not fit,
 * the call takes the float64 dot instead, with the same tokens.  Errors: as
 * ce_top_tokens, plus UNSUPPORTED when even that workspace exceeds
 * CE_STATIC_SCRATCH_BYTES, HIP if the array's address cannot be found. */
#define CE_STATIC_SCRATCH_BYTES (4u << 20)
ce_status ce_top_tokens_static(ce_head_t head, const void* h, int32_t B, int32_t K,
                               int32_t* tokens, int32_t* topk_ids_or_null,
                               hipStream_t stream);

/* forward: logits[b][t] = canonical logit of token t if t is owned by one of
 * row b's K selected centroids, else -inf.  Every entry of [B][V] is written.
 *   logits  DEVICE [B][V] fp32, 16-byte aligned
 * Other arguments and errors as ce_top_tokens. */
ce_status ce_masked_logits(ce_head_t head, const void* h, int32_t B, int32_t K,
                           float* logits, int32_t* topk_ids_or_null, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* Fused top-m over the candidates, the step after get_top_tokens that tree
 * drafting and sampling need (next step named with the page's argmax): for
 * every row b < B, the m candidate tokens (those owned by the row's K
 * selected centroids) with the largest canonical logits, ordered by logit
 * descending then token id ascending, and their fp32 logits, without
 * building the full-vocabulary row.  A row with fewer than m candidates is
 * padded with token -1 and logit -inf.
 *   m        1..CE_MAX_TOP_M
 *   tokens   DEVICE [B][m] int32
 *   logits   DEVICE [B][m] fp32
 *   ws       DEVICE workspace of ce_workspace_bytes(head, B, K, CE_OP_TOP_M)
 *            (the same for every m), 256-byte aligned
 * Other arguments and errors as ce_top_tokens, plus BAD_SHAPE for m out of
 * range and UNSUPPORTED when a row's K largest clusters hold too many tiles
 * for the merge (more than 8160 - 64*m tiles of 64 tokens: 6112 at m = 32,
 * 7648 at m = 8). */
#define CE_MAX_TOP_M 32
ce_status ce_top_m(ce_head_t head, const void* h, int32_t B, int32_t K, int32_t m,
                   int32_t* tokens, float* logits, int32_t* topk_ids_or_null,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/* ce_top_m with each candidate's log-probability under the softmax over the
 * row's candidate set in place of its logit: the softmax a sampler takes
 * over the forward's masked row (vLLM compare view, gemma4_mtp.py,
 * Gemma4MTPMaskedEmbedder.forward: -inf outside the candidates, so those
 * tokens get probability 0), normalised over all the row's candidates, not
 * only the m returned.  With M the row's largest canonical logit and T the
 * sum of exp(l_c - M) over every candidate but one holding M, in float64:
 *   logprobs[b][i] = fp32((l_i - M) - log1p(T)),
 * rounded once to nearest-even; the summation order of T is fixed by the
 * library, so results repeat bit for bit, and they lie within one fp32
 * step of the same formula evaluated exactly.  Tokens and their order are
 * exactly ce_top_m's; padding is token -1 with log-probability -inf.
 *   logprobs  DEVICE [B][m] fp32
 *   ws        DEVICE workspace of ce_workspace_bytes(head, B, K,
 *             CE_OP_TOP_M_LOG_SOFTMAX) (the same as for CE_OP_TOP_M)
 * Other arguments and errors as ce_top_m. */
ce_status ce_top_m_log_softmax(ce_head_t head, const void* h, int32_t B, int32_t K, int32_t m,
                               int32_t* tokens, float* logprobs, int32_t* topk_ids_or_null,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* Fused draft step around the head (the step after the head that fuses its
 * neighbours).  In the page's multi-token predictor (Gemma4MultiTokenPredictor
 * forward) the head scores the output of the final RMSNorm, and the next
 * draft step starts from embed_input_ids: the chosen token's backbone
 * embedding times the float32 `normalizer` buffer.  For every row b < B:
 *   h_out[b]  = RMSNorm(x[b]) with weight norm_weight and epsilon eps:
 *               x_k w_k / sqrt(mean_j x_j^2 + eps) in the canonical norm
 *               rounding: the sum of squares is the float64 chain
 *               ss = fl64(ss + x_k^2) over k in order from +0.0 (squares
 *               exact), then v = ss/d + eps, r = 1/sqrt(v),
 *               y = (x_k r) w_k in correctly rounded float64 steps, y rounded
 *               to float32 and then to the head's dtype (nearest, ties even);
 *   tokens[b] = get_top_tokens of h_out[b], exactly as ce_top_tokens;
 *   emb_out[b] = emb_table[tokens[b]] * normalizer, the float32 product
 *               rounded to the head's dtype; zeros when tokens[b] is -1.
 *               Only when emb_table is not NULL.
 *   x            DEVICE [B][d] rows before the norm, head dtype, 16-byte aligned
 *   norm_weight  DEVICE [d] head dtype, 16-byte aligned
 *   eps          finite, > 0
 *   h_out        DEVICE [B][d] head dtype, 16-byte aligned
 *   tokens       DEVICE [B] int32
 *   emb_table    DEVICE [V][emb_dim] head dtype indexed by token id, 16-byte
 *                aligned, or NULL
 *   emb_dim      > 0, emb_dim * element size a multiple of 16 (with a table)
 *   normalizer   finite float32 scale (with a table)
 *   emb_out      DEVICE [B][emb_dim] head dtype, 16-byte aligned (with a table)
 *   ws           DEVICE workspace of ce_workspace_bytes(head, B, K,
 *                CE_OP_DRAFT_STEP), 256-byte aligned
 * Other arguments and errors as ce_top_tokens, plus BAD_SHAPE for eps,
 * emb_dim or normalizer out of range.  x and h_out must not overlap. */
ce_status ce_draft_step(ce_head_t head, const void* x, const void* norm_weight, float eps,
                        int32_t B, int32_t K, void* h_out, int32_t* tokens,
                        const void* emb_table, int32_t emb_dim, float normalizer,
                        void* emb_out, int32_t* topk_ids_or_null, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* Capture one call into an instantiated HIP graph, the counterpart of the
 * page's per-batch-size CUDA graphs (Gemma4Proposer._setup_centroids_cuda_graphs
 * in the vLLM compare view, diff of spec_decode/gemma4.py).  The graph reads
 * its inputs and writes its outputs and workspace at the addresses given here
 * on every launch; new inputs written there are picked up by the next launch.
 * `stream` must not be the null stream; it is used only for capture.
 * This form covers the ops whose call these arguments describe:
 *   CE_OP_SCORE          h -> out = scores [B][Nc] fp32 (K, topk_ids, ws unused)
 *   CE_OP_TOPK           h = scores [B][Nc] fp32 -> out = topk ids [B][K]
 *                        (topk_ids, ws unused)
 *   CE_OP_TOP_TOKENS     h -> out = tokens [B]
 *   CE_OP_MASKED_LOGITS  h -> out = logits [B][V]
 * and ce_graph_capture_call every op, CE_OP_TOP_M, CE_OP_TOP_M_LOG_SOFTMAX
 * and CE_OP_DRAFT_STEP included.  Errors: as the captured call (checked before anything is
 * enqueued, so a failed call leaves no capture behind), plus UNSUPPORTED for
 * another op or the null stream, HIP for a capture failure. */
ce_status ce_graph_capture(ce_head_t head, int32_t op, const void* h, int32_t B,
                           int32_t K, void* out, int32_t* topk_ids_or_null,
                           void* ws, size_t ws_bytes, hipStream_t stream,
                           ce_graph_t* graph);

/* One call of any compute op, as ce_graph_capture_call takes it.  Each field
 * has the meaning of the same argument of the op's own entry point; fields an
 * op does not take are ignored.
 *   op          ce_op
 *   in          h (SCORE, TOP_TOKENS, MASKED_LOGITS, TOP_M, TOP_M_LOG_SOFTMAX),
 *               the scores (TOPK) or the rows before the norm, x (DRAFT_STEP)
 *   out         scores (SCORE), topk ids (TOPK), tokens (TOP_TOKENS, TOP_M,
 *               TOP_M_LOG_SOFTMAX, DRAFT_STEP) or logits (MASKED_LOGITS)
 *   out_logits  the [B][m] logits of TOP_M, the log-probabilities of
 *               TOP_M_LOG_SOFTMAX
 *   topk_ids    topk_ids_or_null of the fused ops
 *   norm_weight, eps, h_out, emb_table, emb_dim, normalizer, emb_out
 *               the DRAFT_STEP operands */
typedef struct ce_call {
  int32_t op;
  const void* in;
  int32_t B;
  int32_t K;
  int32_t m;
  void* out;
  float* out_logits;
  int32_t* topk_ids;
  void* ws;
  size_t ws_bytes;
  const void* norm_weight;
  float eps;
  void* h_out;
  const void* emb_table;
  int32_t emb_dim;
  float normalizer;
  void* emb_out;
} ce_call;

/* Capture the call `*call` of any op into an instantiated HIP graph, as
 * ce_graph_capture does.  Errors: NULL_POINTER for call or graph, otherwise
 * as ce_graph_capture. */
ce_status ce_graph_capture_call(ce_head_t head, const ce_call* call, hipStream_t stream,
                                ce_graph_t* graph);

/* Launch a captured graph on `stream`.  Errors: NULL_POINTER, HIP. */
ce_status ce_graph_launch(ce_graph_t graph, hipStream_t stream);

/* Destroy a captured graph.  NULL is accepted. */
ce_status ce_graph_destroy(ce_graph_t graph);

/* Measurement hook: the next ce_top_tokens or ce_masked_logits call made by
 * this thread (not under capture) records `start` and `stop` on its stream
 * immediately around the candidate gather kernel, through the HIP extended
 * launch so that the pair brackets that kernel alone.  Consumed by that call.
 * Errors: NULL_POINTER. */
ce_status ce_probe_gather_events(hipEvent_t start, hipEvent_t stop);

/* Measurement probe: enqueue on `stream` one kernel that reads every 16-byte
 * vector of the device buffer buf[0, bytes) once (coalesced, grid-stride,
 * eight independent non-temporal loads in flight per thread: the fastest of
 * the configurations measured), the streaming read rate the gather's
 * bandwidth is compared against.  `sink` is a device word the kernel writes
 * only if the XOR of the data equals an improbable pattern; its content is
 * meaningless.  The caller owns both buffers.
 * Errors: NULL_POINTER, MISALIGNED (buf or bytes not a multiple of 16), HIP. */
ce_status ce_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                               hipStream_t stream);

/* Measurement: of the rows the fused calls have processed with the MFMA
 * projection since ce_head_prepare, counts[0] had the K-th place decided by
 * recomputed canonical keys of the centroids near it, and counts[1] had all
 * their keys recomputed (non-finite sums, masses of near-equal scores).
 * Copies two counters from the persistent buffer and synchronises the
 * device: not for the hot path.  Errors: NULL_POINTER, NOT_PREPARED, HIP. */
ce_status ce_head_repair_counts(ce_head_t head, uint64_t counts[2]);

/* Measurement probe: the MFMA projection alone, scores[b][c] = the matrix
 * cores' fp32 sum of h[b] . centroid c (bf16 heads), the approximate scores
 * whose error bound the certified top-K relies on.  Errors: as
 * ce_score_centroids, plus BAD_DTYPE for an fp32 head. */
ce_status ce_probe_approx_scores(ce_head_t head, const void* h, int32_t B, float* scores,
                                 hipStream_t stream);

/* Short name of a status code.  Never NULL. */
const char* ce_status_string(ce_status status);

/* Message for the calling thread's last failure ("" if none).  Never NULL. */
const char* ce_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CE_H_ */
