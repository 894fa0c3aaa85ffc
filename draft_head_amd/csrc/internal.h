// Host-side declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dh {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kMaxChainGroup = 32;  // sequences per chain launch (two 16-column MFMA blocks)

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
  const float* Lb;         // [B][P][V]
  float* out_logits;       // [B][P][V] or null
  int32_t* out_tokens;     // [B][P]
  const int32_t* t0;       // [B]
  const float* zh;         // [B][P][r]  W1[:, :d] H
  float* h;                // [P+1][h_step] GRU state after each step (slot 0 = zeros)
  void* act;               // [P][act_step bytes] bottleneck activations of each step:
                           //   bf16 hi [B][r] then lo [B][r], or fp32 [B][r]
  uint64_t* keys;          // [P][B] packed argmax keys
  uint32_t* counters;      // [4][sub-counters][line] phase arrival counters
  int32_t* status;         // device status word
  int h_step;              // floats between consecutive state slots (256-byte multiple)
  int act_step;            // bytes between consecutive activation slots (256-byte multiple)
  uint64_t* trace;         // phase timestamps [P][grid][6] when built with DH_TRACE_PHASES, else null
};

// workspace carving for a chain launch of up to `group` sequences
struct ChainLayout {
  size_t status, counters, keys, zh, h, act, trace, total;
  int h_step, act_step;
};
ChainLayout chain_layout(int d, int Hs, int r, int P, int group);

// prologue (H half of the bottleneck, zeroed state) then the P steps
hipError_t launch_chain(int dtype, const ChainArgs& a, const void* H, int mode, bool reset_status, hipStream_t s,
                        hipEvent_t ev_start, hipEvent_t ev_stop);

}  // namespace dh
