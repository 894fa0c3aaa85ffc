// Host-side declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dh {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kMaxChainGroup = 32;  // sequences per chain launch (two 16-column MFMA blocks)
constexpr int kMaxChainGrid = 1024; // workgroups of a persistent chain launch at most
constexpr int kMaxZhSplits = 8;     // k splits of the H half of the bottleneck at most
// device-side status word at offset 0 of a workspace
constexpr int kDeviceStatusFirstToken = 1;  // a first token outside [0, V) was replaced by 0
constexpr int kDeviceStatusTimeout = 2;     // a wait between workgroups gave up

// compute units of the current device (0 if the query fails)
inline int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 0;
  return cus;
}

// C[m][n] = sum_k A[m][k] B[n][k], fp32 out.  prefer_tiles selects the
// LDS-tiled kernel for many rows of A (bf16 only).
hipError_t launch_gemm_nt(int dtype, const void* A, int lda, const void* B, int ldb, float* C, int ldc, int M, int N,
                          int K, bool prefer_tiles, hipStream_t s);

// Everything one chain launch needs; device pointers.
struct ChainArgs {
  int d, V, Hs, r, P, B;  // B = sequences in this launch (<= kMaxChainGroup)
  const void* embed;
  const void* w_ih;
  const void* w_hh;
  const void* w1;
  const void* w2;
  const float* b_ih;
  const float* b_hh;
  const float* b1;
  const float* b2;
  const float* xt;         // [V][3 Hs] W_ih E[v] per token (input half of the GRU), or null: computed from embed and w_ih
  const float* Lb;         // [B][P][V]
  float* out_logits;       // [B][P][V] or null
  int32_t* out_tokens;     // [B][P]
  const int32_t* t0;       // [B]
  const float* zh;         // [zh_splits][B][P][r]  W1[:, :d] H, as partial sums over k splits
  int zh_splits;           // partial sums in zh (added in split order by the bottleneck)
  int zh_stride;           // floats between consecutive partials
  float* zh_sum;           // [B][P][r] the partials added, written by the persistent launch's bottleneck workgroups
  float* h;                // [P+1][h_step] GRU state after each step (slot 0 = zeros)
  uint16_t* hb;            // [P+1][hb_step] the same states split for bf16 MFMA: hi [B][Hs], lo [B][Hs]
  void* act;               // [P][act_step bytes] bottleneck activations of each step:
                           //   bf16 hi [B][r] then lo [B][r], or fp32 [B][r]
  uint64_t* keys;          // [P][B] packed argmax keys
  int32_t* status;         // device status word
  int h_step;              // floats between consecutive state slots (256-byte multiple)
  int hb_step;             // bf16 elements between consecutive split-state slots (256-byte multiple)
  int act_step;            // bytes between consecutive activation slots (256-byte multiple)
  uint64_t* trace;         // phase timestamps [P][grid][slots] when built with DH_TRACE_PHASES, else null
  // tagged hand-off words of the persistent schedule
  uint64_t* ll_h;          // [P+1][B][Hs] state after each step (bf16: hi pairs, then lo pairs; fp32: one per word)
  uint64_t* ll_act;        // [P][B][r] bottleneck activations, same packing
  uint64_t* ll_part;       // [P][kMaxChainGrid][B][2] each workgroup's argmax (value, index) per sequence
  uint64_t* ll_tok;        // [P][B][2] per-sequence argmax when reduced in two levels
  uint32_t* epoch;         // launch counter, advanced by the prologue
  uint64_t* marker;        // kLLMarker once the hand-off words have been cleared
  uint64_t* sig;           // layout signature the hand-off words were cleared for
  uint64_t sig_value;      // this launch's layout signature
  size_t ll_words;         // hand-off words from ll_h on (all four regions)
  uint64_t* stamps;        // [P+1] step start clocks of the persistent schedule (first workgroup)
  // sampling: the token is argmax (L + temperature * Gumbel noise) when temperature > 0
  float temperature;
  uint32_t seed_lo, seed_hi;
  int seq_base;            // index of this launch's first sequence in the whole batch (a multiple of 32)
};

// workspace carving for a chain launch of up to `group` sequences
struct ChainLayout {
  size_t status, stamps, keys, zh, zh_sum, h, hb, act, ll_h, ll_act, ll_part, ll_tok, trace, total;
  int h_step, hb_step, act_step;
};
ChainLayout chain_layout(int d, int Hs, int r, int P, int group);
// k splits of the H half for a launch of B sequences
int zh_splits(int d, int r, int P, int B);
// frees the per-device events that order persistent launches
void release_chain_cache();

// prologue (H half of the bottleneck, zeroed state) then the P steps
hipError_t launch_chain(int dtype, const ChainArgs& a, const void* H, int mode, bool reset_status, hipStream_t s,
                        hipEvent_t ev_start, hipEvent_t ev_stop);

// Everything one tree call needs; device pointers.
struct TreeArgs {
  int d, V, Hs, r, P, B, N, M, dtype;
  const void* H;
  const void* embed;
  const void* w_ih;
  const void* w_hh;
  const void* w1;
  const void* w2;
  const float* b_ih;
  const float* b_hh;
  const float* b1;
  const float* b2;
  const double* xt;         // [V][3 Hs] W_ih E[v] per token in fp64 (input half of the GRU), or null
  const float* Lb;          // [B][P][V]
  const int32_t* t0;        // [B]
  int32_t* out_parents;     // [B][N]
  int32_t* out_tokens;      // [B][N]
  int32_t* out_depth;       // [B][N] or null
  double* out_scores;       // [B][N] or null
  uint64_t* seg_keys;       // [B*P][segments][M] per-segment top-M keys
  int32_t* cand_idx;        // [B][P][M] top-M candidates per row
  float* cand_val;          // [B][P][M]
  double* zh;               // [B][P][r] W1[:, :d] H in fp64
  double* zh_cur;           // [B][r] the row of zh at the depth of the node each sequence expands next
  double* act;              // [B][r] bottleneck of the node being expanded, fp64
  double* states;           // [B][N+1][Hs] fp64 GRU state per node (slot 0 = anchor)
  double* gh;               // [B][N+1][3][Hs] W_hh h of each node's state (one launch per round with the table)
  double* heap_score;       // [B][heap_cap]
  int4* heap_meta;          // [B][heap_cap] (parent, rank, token, depth)
  int32_t* heap_count;      // [B]
  void* cur;                // [B] node being expanded this round
  int32_t* status;
  int heap_cap;
  // tagged hand-off words of the one-launch-per-round schedule (bf16 weights)
  uint64_t* ll_act;         // [N][B][r][2] the bottleneck of each round, fp64 as two 32-bit halves
  uint64_t* ll_cur;         // [N][B][2] each round's popped node: token; parent slot + 1 | expand << 16
  uint32_t* epoch;          // call counter, advanced by tree_init
  uint64_t* marker;         // kLLMarker once the hand-off words have been cleared
  uint64_t* sig;            // layout signature the hand-off words were cleared for
  uint64_t sig_value;       // this call's layout signature
  size_t ll_words;          // hand-off words from ll_act on (both regions)
};

struct TreeLayout {
  size_t status, seg_keys, cand_idx, cand_val, zh, zh_cur, act, states, gh, heap_score, heap_meta, heap_count, cur, ll_act,
      ll_cur, total;
  int heap_cap;
};
TreeLayout tree_layout(int d, int Hs, int r, int P, int group, int N, int M);

hipError_t launch_tree(const TreeArgs& t, bool reset_status, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop);
// table[v][g] = sum_k E[v][k] Wih[g][k] in fp64 for v < V, g < 3 Hs
hipError_t launch_input_table_f64(int dtype, const void* E, const void* Wih, int V, int Hs, int d, double* table,
                                  hipStream_t s);
// dynamic LDS of the tree's GRU kernel (must stay within the CU's 160 KB)
size_t tree_gru_lds(int d, int Hs, int dtype);
size_t tree_gru_lds_total(int d, int Hs, int dtype);  // the GRU step's whole LDS (160 KB per CU)
// top-M of each of `rows` rows of length V, ordered (value desc, index asc);
// scratch holds topm_scratch_bytes(rows, M)
size_t topm_scratch_bytes(int rows, int M);
hipError_t launch_topm(const float* Lb, int rows, int V, int M, void* scratch, int32_t* idx, float* val, hipStream_t s);

// verification inputs of B flattened trees of N nodes (verify.hip)
hipError_t launch_tree_verify_inputs(const int32_t* parents, const int32_t* tokens, const int32_t* first_tokens,
                                     const int32_t* start_positions, int B, int N, uint8_t* mask, int32_t* positions,
                                     int32_t* out_tokens, hipStream_t s);

}  // namespace dh
