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
 *   - Errors: a non-zero domino_status is returned and domino_last_error()
 *     (per thread) describes it.  No C++ exception crosses the ABI.
 *   - Calls are stateless and may run concurrently on distinct streams with
 *     distinct workspaces and outputs.  The persistent chain schedule keeps a
 *     workgroup on every CU for the whole call; the library orders such
 *     launches one after another on each device, whatever their streams.
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
  DOMINO_ERR_INVALID_ARGUMENT = 1, /* null / misaligned pointer, bad dimension or count */
  DOMINO_ERR_UNSUPPORTED = 2,      /* valid but outside what the kernels implement     */
  DOMINO_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required        */
  DOMINO_ERR_DEVICE = 4            /* a HIP runtime call failed; see domino_last_error  */
} domino_status;

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
} domino_weights;

/* Library version string (static storage). */
const char *domino_version(void);

/* Message for the last non-OK status returned on the calling thread
 * (static thread-local storage; "" when none). */
const char *domino_last_error(void);

/*
 * Base logits (device):  base_logits[b][p][v] = sum_k H[b][p][k] * lm_head[v][k]
 * for b < batch, p < block, v < vocab, computed with fp32 accumulation and
 * stored fp32.  H is [batch][block][hidden] in dims.dtype.  batch == 0 is a
 * no-op.  The contraction runs on the MFMA matrix cores.
 */
domino_status domino_base_logits(const domino_dims *dims, const domino_weights *weights, const void *H,
                                 int32_t batch, float *base_logits, void *stream);

/* Bytes of workspace domino_draft_chain needs for `batch` sequences. */
size_t domino_chain_workspace_size(const domino_dims *dims, int32_t batch);

/*
 * The sequential correction chain over one draft block for `batch`
 * independent sequences.  For position p = 0..P-1 and each sequence:
 *   h    = GRU(embed[prev], h)       prev = first_tokens[b] at p = 0, else the token drafted at p-1
 *   a    = SiLU(W1 [H[b][p] ; h] + b1)
 *   L    = base_logits[b][p] + W2 a + b2
 *   out_tokens[b][p] = argmax_v L   (lowest index among equal maxima; -0 == +0)
 * Inputs (device): H [batch][P][d]; base_logits [batch][P][V] fp32 (normally
 *   the output of domino_base_logits); first_tokens [batch] int32 in [0, V).
 * Outputs (device): out_tokens [batch][P] int32; out_logits [batch][P][V]
 *   fp32 final logits, or NULL to skip them (may equal base_logits for an
 *   in-place update).
 * workspace (device): at least domino_chain_workspace_size(dims, batch)
 *   bytes.  After the call completes, the int32 at offset 0 of the workspace
 *   holds a device-side status: 0 = fine, 1 = a first token was outside
 *   [0, V) (that sequence was drafted from token 0 instead), 2 = an internal
 *   wait timed out (outputs undefined).
 * batch == 0 is a no-op.  Calls that share a workspace must not overlap.
 */
domino_status domino_draft_chain(const domino_dims *dims, const domino_weights *weights, const void *H,
                                 const float *base_logits, const int32_t *first_tokens, int32_t batch,
                                 int32_t *out_tokens, float *out_logits, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* Bytes of workspace domino_tree_candidates needs (0 for invalid arguments). */
size_t domino_tree_candidates_workspace_size(const domino_dims *dims, int32_t batch, int32_t topm);

/*
 * Top-M candidates of every base-logit row (the tree's candidate lists,
 * DominoTree summary, "Top-M" restriction): for each of batch*block rows of
 * base_logits [batch][block][vocab] (device, fp32), out_index/out_value
 * [batch][block][topm] (device) hold the topm largest entries ordered by
 * (value desc, index asc); -0.0 counts as +0.0.  1 <= topm <= min(256, vocab).
 * workspace (device): domino_tree_candidates_workspace_size bytes of scratch.
 */
domino_status domino_tree_candidates(const domino_dims *dims, const float *base_logits, int32_t batch, int32_t topm,
                                     int32_t *out_index, float *out_value, void *workspace, size_t workspace_bytes,
                                     void *stream);

/* Bytes of workspace domino_tree_draft needs (0 for invalid arguments). */
size_t domino_tree_workspace_size(const domino_dims *dims, int32_t batch, int32_t nodes, int32_t topm);

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
 * The int32 at workspace offset 0 holds the device status after the call
 * (1 = a first token was outside [0, V) and token 0 was used).
 */
domino_status domino_tree_draft(const domino_dims *dims, const domino_weights *weights, const void *H,
                                const float *base_logits, const int32_t *first_tokens, int32_t batch, int32_t nodes,
                                int32_t topm, int32_t *out_parents, int32_t *out_tokens, int32_t *out_depth,
                                double *out_scores, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Timing hooks for benchmarks and profilers (hipEvent_t handles passed as
 * void*).  While set, each later domino_base_logits call records base_start
 * on its stream right before its GEMM launch and base_stop right after it,
 * and each domino_draft_chain call records chain_start right before the
 * launch(es) that run the P steps (after the short prologue) and chain_stop
 * right after them; each domino_tree_draft call records the chain pair around
 * all of its launches.  A NULL pair disables that pair.  The events stay owned
 * by the caller.  Process-wide setting; not for concurrent callers.
 */
void domino_set_timing_events(void *base_start, void *base_stop, void *chain_start, void *chain_stop);

/*
 * Chain scheduling.  0 (default): the library picks; for up to 8 sequences
 * one persistent launch runs all P steps and, for bf16 weights
 * where it fits, keeps W2 on chip (registers and LDS) for all of them; for
 * more sequences, three kernel launches per step.  1: three launches per
 * step.  2: the persistent launch with W2 read from memory every step.  All
 * compute the same function with the same summation order, so their outputs
 * agree to the bit.  Returns the previous mode; any other value is rejected
 * with -1.  Process-wide setting.
 */
int32_t domino_set_chain_mode(int32_t mode);

#ifdef __cplusplus
}
#endif

#endif /* DOMINO_H */
