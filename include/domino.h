/*
 * domino.h — C ABI of the Domino draft-head hot path on MI355X (gfx950).
 *
 * The Domino draft head turns one parallel-drafted block of P positions into
 * P drafted tokens in two parts:
 *   1. block-parallel base logits  Lb_i = H_i W_lm^T  through the frozen LM
 *      head, all positions at once (Domino paper summaries: Dutch gist.science
 *      page, "Methodologie: Domino", part 1; 163.com explainer, section 3);
 *   2. a sequential causal-correction chain: a GRU reads the embedding of the
 *      previously drafted token, W1 projects [H_i ; S] to a rank-r bottleneck,
 *      SiLU, W2 projects back to the vocabulary, the correction is added in
 *      logit space, L_i = Lb_i + dL_i, and the greedy token is the argmax
 *      (Dutch page, part 2 "Domino-head"; explainer, section 4; Korean review
 *      dimensionstp.github.io, section 3-2 and its final-logits equation).
 * A best-first tree variant scores children of every node with that node's
 * own GRU state, restricted to the top-M base-logit candidates of each depth
 * (DominoTree summary, gist.science Chinese page, technical abstract,
 * "方法论": conditional best-first heap; Top-M candidate restriction).
 *
 * Conventions shared by every call
 *   - Every pointer argument marked (device) is device memory owned by the
 *     caller; the library never frees, keeps or allocates such memory.
 *     Every device pointer must be 16-byte aligned.
 *   - All arrays are dense, row-major, C-contiguous.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream.  Calls only enqueue work: outputs are valid once the stream
 *     has reached that point.  Nothing is written before validation passes.
 *   - Storage type (`dims.dtype`): DOMINO_BF16 (H and all weight matrices
 *     bf16) or DOMINO_F32 (all fp32).  Biases are always fp32 and optional
 *     (NULL = zero).  Arithmetic is fp32 with fp32 accumulation; the tree's
 *     scoring is fp64.
 *   - The GRU follows the torch.nn.GRUCell form with gate blocks (r, z, n):
 *       r = s(W_ir x + b_ir + W_hr h + b_hr), z = s(W_iz x + b_iz + W_hz h + b_hz),
 *       n = tanh(W_in x + b_in + r (W_hn h + b_hn)), h' = (1 - z) n + z h,
 *     starting from h = 0 and reading the anchor token first.
 *   - Errors: a negative domino_status is returned and domino_last_error()
 *     (per thread) describes it.  No C++ exception crosses the ABI.
 *   - Device-side status.  Conditions found while the kernels run (a first
 *     token outside [0, V), a wait between workgroups that gave up) cannot be
 *     returned by the enqueueing call.  The kernels write them to the int32 at
 *     offset 0 of the call's workspace; domino_device_status() waits for the
 *     stream and turns that word into a domino_status.  A caller that skips
 *     it must treat the outputs of a call whose word reads 2 as undefined.
 *   - Concurrency.  The library keeps no state that changes the results of a
 *     call.  Calls may run concurrently on distinct streams with distinct
 *     workspaces and outputs.  The chain's one-launch schedule keeps a
 *     workgroup on every CU for the whole call and its workgroups wait for
 *     each other; the library orders such launches one after another on each
 *     device, whatever their streams (one HIP event per device, kept until
 *     domino_release_cache).  A device whose CUs are partly held by other
 *     work (another process, a CU-masked stream) can make those waits give
 *     up after 2 s: the call then reports DOMINO_ERR_TIMEOUT through
 *     domino_device_status.
 *   - Benchmark and test hooks that change process-wide settings live in
 *     domino_bench.h, outside this contract.
 */
#ifndef DOMINO_H
#define DOMINO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DOMINO_OK = 0,
  DOMINO_ERR_INVALID_ARGUMENT = -1, /* null / misaligned pointer, bad dimension or count  */
  DOMINO_ERR_UNSUPPORTED = -2,      /* valid but outside what the kernels implement      */
  DOMINO_ERR_WORKSPACE = -3,        /* workspace missing or smaller than required         */
  DOMINO_ERR_DEVICE = -4,           /* a HIP runtime call failed; see domino_last_error   */
  DOMINO_ERR_TIMEOUT = -5,          /* (domino_device_status) a wait between workgroups
                                       gave up: the outputs of that call are undefined   */
  DOMINO_ERR_FIRST_TOKEN = -6       /* (domino_device_status) a first token was outside
                                       [0, V); that sequence was drafted from token 0    */
} domino_status;

/* The call domino_workspace_size is asked about. */
typedef enum {
  DOMINO_OP_BASE = 0,      /* domino_base_logits: needs no workspace (size 0)        */
  DOMINO_OP_CHAIN = 1,     /* domino_draft_chain and domino_draft_chain_sampled       */
  DOMINO_OP_TREE = 2,      /* domino_tree_draft                                       */
  DOMINO_OP_CANDIDATES = 3 /* domino_tree_candidates                                  */
} domino_op;

typedef enum { DOMINO_F32 = 0, DOMINO_BF16 = 1 } domino_dtype;

/* Model dimensions.  hidden, gru_hidden and rank must be multiples of 8;
 * rank <= 256; 1 <= block <= 64; vocab >= 1. */
typedef struct {
  int32_t hidden;     /* d:  backbone hidden size                      */
  int32_t vocab;      /* V:  vocabulary size                           */
  int32_t gru_hidden; /* Hs: GRU state width (1024 on the pages)       */
  int32_t rank;       /* r:  correction bottleneck (256 on the pages)  */
  int32_t block;      /* P:  positions per draft block (16)            */
  int32_t dtype;      /* domino_dtype of H and of every weight matrix  */
} domino_dims;

/* Weights (device).  Gate blocks of w_ih / w_hh are stacked (r, z, n). */
typedef struct {
  const void *lm_head; /* [V][d]     frozen target LM head                  */
  const void *embed;   /* [V][d]     token embedding read by the GRU (may alias lm_head) */
  const void *w_ih;    /* [3Hs][d]                                          */
  const void *w_hh;    /* [3Hs][Hs]                                         */
  const float *b_ih;   /* [3Hs] or NULL                                     */
  const float *b_hh;   /* [3Hs] or NULL                                     */
  const void *w1;      /* [r][d+Hs]  columns 0..d-1 act on H_i, d.. on S    */
  const float *b1;     /* [r] or NULL                                       */
  const void *w2;      /* [V][r]                                            */
  const float *b2;     /* [V] or NULL                                       */
  const float *input_table; /* [V][3Hs] fp32 from domino_prepare_input_table,
                        * or NULL; used by the chain calls only          */
  const double *input_table_f64; /* [V][3Hs] fp64 from
                        * domino_prepare_input_table_f64, or NULL; used by
                        * domino_tree_draft only                         */
} domino_weights;

/* Library version string (static storage). */
const char *domino_version(void);

/* Message for the last non-OK status returned on the calling thread
 * (static thread-local storage; "" when none). */
const char *domino_last_error(void);

/*
 * Bytes of device workspace a call needs: `op` is a domino_op; `nodes` and
 * `topm` matter for DOMINO_OP_TREE (both) and DOMINO_OP_CANDIDATES (topm)
 * only.  Returns 0 for DOMINO_OP_BASE and for arguments the call would reject
 * (then domino_last_error says why).  A workspace sized for `batch`
 * sequences serves any smaller batch of the same dims.
 */
size_t domino_workspace_size(const domino_dims *dims, int32_t batch, int32_t op, int32_t nodes, int32_t topm);

/*
 * Device status of the last call that used `workspace` (device): waits for
 * `stream` (which must be the stream of that call, or one ordered after it),
 * reads the int32 at offset 0 and returns DOMINO_OK (0), DOMINO_ERR_FIRST_TOKEN
 * (1) or DOMINO_ERR_TIMEOUT (2); DOMINO_ERR_DEVICE if the wait or the read
 * fails.  The word is reset by the next call that uses the workspace.
 */
domino_status domino_device_status(const void *workspace, void *stream);

/*
 * Releases what the library keeps for the life of the process: the event that
 * orders one-launch chain schedules on each device, and the cached launch
 * settings of the calling thread.  Waits for that event first.  Safe to call
 * at any time when no call is being enqueued; later calls recreate what they
 * need.
 */
void domino_release_cache(void);

/*
 * Base logits (device):  base_logits[b][p][v] = sum_k H[b][p][k] * lm_head[v][k]
 * for b < batch, p < block, v < vocab, computed with fp32 accumulation and
 * stored fp32.  H is [batch][block][hidden] in dims.dtype.  batch == 0 is a
 * no-op.  The contraction runs on the MFMA matrix cores.
 */
domino_status domino_base_logits(const domino_dims *dims, const domino_weights *weights, const void *H,
                                 int32_t batch, float *base_logits, void *stream);

/*
 * The GRU's input half for every token, once per set of weights (the GRU
 * reads the embedding of the previous drafted token: 163.com explainer,
 * section 4, causal encoder; Dutch Domino summary, "Methodologie", part 2):
 *   table[v][g] = sum_k embed[v][k] * w_ih[g][k]   for v < vocab, g < 3 gru_hidden
 * with fp32 accumulation, stored fp32 (row v holds the r, z and n blocks of
 * W_ih embed[v]).  table is caller-owned device memory of
 * vocab * 3 * gru_hidden floats (1.87 GB at V = 151936, gru_hidden = 1024).
 * Passed as weights.input_table to the chain calls, it replaces their
 * W_ih x product: each step then reads one table row per sequence instead of
 * an embedding row and all of w_ih.  embed and w_ih are read here only; the
 * table must be rebuilt when either changes.  Uses weights.embed and
 * weights.w_ih; the other weight pointers are not read.  Runs on the MFMA
 * matrix cores (about 2.4 TFLOP at the Qwen3-4B shapes).
 */
domino_status domino_prepare_input_table(const domino_dims *dims, const domino_weights *weights, float *table,
                                        void *stream);

/*
 * The same table in fp64 for the tree, whose GRU and scores run in fp64:
 *   table[v][g] = sum_k embed[v][k] * w_ih[g][k]   (products exact, fp64 sums)
 * for v < vocab, g < 3 gru_hidden; table is caller-owned device memory of
 * vocab * 3 * gru_hidden doubles (3.73 GB at V = 151936, gru_hidden = 1024).
 * Passed as weights.input_table_f64 to domino_tree_draft, it replaces the
 * tree GRU's W_ih x product (one table row per expanded node instead of an
 * embedding row and all of w_ih).  Uses weights.embed and weights.w_ih only;
 * runs on the fp64 matrix cores (about 2.4 TFLOP at the Qwen3-4B shapes).
 */
domino_status domino_prepare_input_table_f64(const domino_dims *dims, const domino_weights *weights, double *table,
                                            void *stream);

/*
 * The sequential correction chain over one draft block for `batch`
 * independent sequences.  For position p = 0..P-1 and each sequence:
 *   h    = GRU(embed[prev], h)       prev = first_tokens[b] at p = 0, else the token drafted at p-1
 *          (with weights.input_table: its row prev as W_ih embed[prev])
 *   a    = SiLU(W1 [H[b][p] ; h] + b1)
 *   L    = base_logits[b][p] + W2 a + b2
 *   out_tokens[b][p] = argmax_v L   (lowest index among equal maxima; -0 == +0)
 * Inputs (device): H [batch][P][d]; base_logits [batch][P][V] fp32 (normally
 *   the output of domino_base_logits); first_tokens [batch] int32 in [0, V).
 * Outputs (device): out_tokens [batch][P] int32; out_logits [batch][P][V]
 *   fp32 final logits, or NULL to skip them (may equal base_logits for an
 *   in-place update).
 * workspace (device): at least domino_workspace_size(dims, batch,
 *   DOMINO_OP_CHAIN, 0, 0) bytes; its device status (domino_device_status):
 *   1 = a first token was outside [0, V) (that sequence was drafted from
 *   token 0 instead), 2 = a wait between workgroups gave up (outputs
 *   undefined).
 * batch == 0 is a no-op.  Calls that share a workspace must not overlap.
 */
domino_status domino_draft_chain(const domino_dims *dims, const domino_weights *weights, const void *H,
                                 const float *base_logits, const int32_t *first_tokens, int32_t batch,
                                 int32_t *out_tokens, float *out_logits, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * The correction chain with every token drawn at temperature T >= 0 instead
 * of taken greedily (the pages report decoding at T = 1 next to greedy
 * decoding: 163.com explainer, section 6; Korean review, section 5;
 * DominoTree summary, experiments at T in {0, 0.5, 1}).  Everything is as in
 * domino_draft_chain except the token of each position, which is the
 * Gumbel-max draw from softmax(L / T):
 *   out_tokens[b][p] = argmax_v (L[b][p][v] + T g(seed, b, p, v))
 * (lowest index on exact ties), fed back to the GRU like the greedy token.
 * g is standard Gumbel noise, -log(-log u), u = (2 (x >> 9) + 1) / 2^24,
 * x = word (b & 1) of Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011)
 * at counter (v, p, b >> 1, 0) under the key (seed & 0xffffffff, seed >> 32);
 * b is the sequence's index in this call.  out_logits, if not NULL, are the
 * unperturbed L.  T = 0 is the greedy chain.  The draws run in the chain's
 * one-launch schedule where W2 stays on chip (bf16, up to 8 sequences), else
 * in the stepwise schedule (two or three launches per step); both draw the
 * same tokens.  temperature must be
 * finite and >= 0.
 */
domino_status domino_draft_chain_sampled(const domino_dims *dims, const domino_weights *weights, const void *H,
                                         const float *base_logits, const int32_t *first_tokens, int32_t batch,
                                         float temperature, uint64_t seed, int32_t *out_tokens, float *out_logits,
                                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * domino_draft_chain without a workspace argument and without allocating:
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * workspace is a static 32 MiB array in the library's code object, one per
 * device, held until the process ends; its address on each device is looked
 * up on the first call on that device.  Every call on a device shares that
 * device's array: calls that overlap on one device (on any streams) race and
 * must not be issued.  Arguments, outputs and results are those of
 * domino_draft_chain.  Returns DOMINO_ERR_UNSUPPORTED when the call needs
 * more than 32 MiB of workspace (domino_workspace_size(dims, batch,
 * DOMINO_OP_CHAIN, 0, 0) > 33554432; Qwen3-4B shapes at batch 32 and block
 * 16 need about 20 MB).  The device status of the last call is read with
 * domino_noalloc_device_status.
 */
domino_status domino_draft_chain_noalloc(const domino_dims *dims, const domino_weights *weights, const void *H,
                                         const float *base_logits, const int32_t *first_tokens, int32_t batch,
                                         int32_t *out_tokens, float *out_logits, void *stream);

/* domino_device_status of the static workspace of domino_draft_chain_noalloc
 * on the current device. */
domino_status domino_noalloc_device_status(void *stream);

/*
 * Top-M candidates of every base-logit row (the tree's candidate lists,
 * DominoTree summary, "Top-M" restriction): for each of batch*block rows of
 * base_logits [batch][block][vocab] (device, fp32), out_index/out_value
 * [batch][block][topm] (device) hold the topm largest entries ordered by
 * (value desc, index asc); -0.0 counts as +0.0.  1 <= topm <= min(256, vocab).
 * workspace (device): domino_workspace_size(dims, batch,
 * DOMINO_OP_CANDIDATES, 0, topm) bytes of scratch.
 */
domino_status domino_tree_candidates(const domino_dims *dims, const float *base_logits, int32_t batch, int32_t topm,
                                     int32_t *out_index, float *out_value, void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * Best-first draft tree with path-conditioned scoring (DominoTree summary,
 * gist.science Chinese page, technical abstract, "方法论 / 核心组件": the
 * conditional best-first heap and the top-M candidate restriction), for
 * `batch` independent sequences.
 *   - Candidates of depth delta (1-based) are the top `topm` entries of
 *     base_logits[b][delta-1], ordered by (value desc, index asc).
 *   - The anchor first_tokens[b] is the root (not counted); its GRU state is
 *     GRU(embed[t0], 0).  Expanding a node at depth delta with state S scores
 *     its topm children on row delta:
 *       l_j = base_logits[b][delta][C_j] + (W2 a)[C_j] + b2[C_j],
 *       a = SiLU(W1 [H[b][delta] ; S] + b1),
 *       child score = node score + l_j - logsumexp_j(l)
 *   - The entry with the highest score is popped next (ties: lower parent
 *     index, then lower candidate rank) and becomes node k = 0, 1, ...; it
 *     gets state GRU(embed[token], S_parent) and is expanded unless it sits at
 *     depth P or is the last node of the budget.
 *   - GRU, bottleneck and scores are fp64.
 * Outputs (device) [batch][nodes]: out_parents (node index, -1 = anchor),
 *   out_tokens, out_depth (1-based; may be NULL), out_scores (fp64; may be
 *   NULL).  Nodes are numbered in pop order, so parents[k] < k.  Slots left
 *   when the tree runs out of nodes hold parent -1, token -1, depth 0,
 *   score -inf.
 * Limits: 1 <= nodes <= 64, 1 <= topm <= min(256, vocab), gru_hidden <= 4096,
 * and, for fp32 weights only, the GRU step's LDS within 160 KB: eight fp64
 * state rows and eight embedding rows (64*gru_hidden + 32*hidden + 256
 * bytes).  The bf16 GRU step reads its operands directly and has no such
 * limit.
 * workspace (device): domino_workspace_size(dims, batch, DOMINO_OP_TREE,
 * nodes, topm) bytes; device status 1 = a first token was outside [0, V)
 * and token 0 was used; 2 = with bf16 weights, where each round runs as one
 * launch whose workgroups hand results to higher-numbered ones through the
 * workspace, such a wait gave up after 2 s (the outputs are then undefined).
 * Calls on one workspace must not overlap.
 */
domino_status domino_tree_draft(const domino_dims *dims, const domino_weights *weights, const void *H,
                                const float *base_logits, const int32_t *first_tokens, int32_t batch, int32_t nodes,
                                int32_t topm, int32_t *out_parents, int32_t *out_tokens, int32_t *out_depth,
                                double *out_scores, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Verification inputs of drafted trees: the standard tree-attention input
 * with an ancestor-only mask that DominoTree keeps for verification
 * (DominoTree summary, "方法论 / 核心组件", verification), for `batch` trees
 * of `nodes` slots as domino_tree_draft writes them.
 * Inputs (device): parents, tokens [batch][nodes] int32 (pop order, -1 for
 *   the anchor / unfilled); first_tokens [batch]; start_positions [batch]
 *   (position id of each anchor) or NULL for 0.
 * Outputs (device), over the flattened entries e = 0 (anchor) and e = k + 1
 *   (node k), E = nodes + 1 per sequence:
 *   out_mask [batch][E][E] uint8: 1 where entry j is entry i itself or one
 *     of its ancestors (the anchor is an ancestor of every tree node);
 *   out_positions [batch][E]: start + depth (anchor 0);
 *   out_tokens [batch][E]: the anchor token, then the node tokens.
 * Node k counts as part of the tree when its token is >= 0 and its parent is
 * the anchor or an earlier node that is part of the tree; any other slot is
 * padding: position -1, token -1, and a mask row with only its own entry.
 * 1 <= nodes <= 64.  Integer work: the result is exact.
 */
domino_status domino_tree_verify_inputs(const int32_t *parents, const int32_t *tokens, const int32_t *first_tokens,
                                        const int32_t *start_positions, int32_t batch, int32_t nodes,
                                        uint8_t *out_mask, int32_t *out_positions, int32_t *out_tokens, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DOMINO_H */
