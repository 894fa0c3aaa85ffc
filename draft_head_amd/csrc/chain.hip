// The sequential causal-correction chain of the Domino head on gfx950.
//
// For every block position p and sequence b (Domino paper summaries: Dutch
// gist.science page, "Methodologie", part 2 "Domino-head"; 163.com
// explainer, section 4; Korean review, section 3-2 final-logits equation):
//   h   = GRU(E[prev], h)               the causal encoder over drafted tokens
//   a   = SiLU(W1 [H_p ; h] + b1)       rank-r bottleneck on the concatenation
//   L   = Lb_p + W2 a + b2              correction added in logit space
//   tok = argmax L                      greedy draft token, fed back as prev
//
// One step is three data-parallel phases with a dependency between each:
//   G  GRU step.  Work item = 4 GRU units.  Its 16 MFMA rows are the 4 units'
//      r, z, n(input half), n(hidden half) pre-activations, so one 16x16 tile
//      yields everything the gate nonlinearity needs and h' is finished in
//      the same workgroup.  k is split over the 4 waves and summed in LDS.
//   W  bottleneck.  Work item = 16 rows of W1's state half; the H half,
//      W1[:, :d] H_p, is computed for all positions before the chain.  The
//      output is written as a bf16 hi + lo pair ready for phase O.
//   O  W2 + base add + argmax.  Each workgroup streams a contiguous range of
//      16-row W2 tiles, keeps the bottleneck fragments in registers, adds the
//      base-logit row in the MFMA epilogue and folds (value, index) into one
//      64-bit key per sequence: wave shuffles, then LDS, then one device-wide
//      atomic max per workgroup.  Full logits are written only on request.
// The drafted token never leaves the device: phase G of the next step reads
// the winning key.
//
// Two schedules compute identical values:
//  * persistent: one cooperative launch for all P steps; phases are
//    separated by arrival counters with bounded waits;
//  * stepwise: three launches per step on the caller's stream.
#include "device.h"
#include "internal.h"

namespace dh {

// Opt-in phase timestamps (constant 100 MHz clock) for tuning builds only.
[[maybe_unused]] constexpr int kTraceSlots = 12;
#ifdef DH_TRACE_PHASES
#define DH_STAMP(p, slot) \
  do { if (a.trace && threadIdx.x == 0) a.trace[((size_t)(p) * gridDim.x + blockIdx.x) * kTraceSlots + (slot)] = wall_clock64(); } while (0)
#else
#define DH_STAMP(p, slot) \
  do { } while (0)
#endif

// Lane index through an opaque move.  Every per-lane address a phase derives
// from it is then recomputed inside the step loop instead of being hoisted
// out of it as a live 64-bit value, which would cost two registers for the
// whole kernel each.
__device__ __forceinline__ int opaque_lane() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}

__device__ __forceinline__ float bias_at(const float* b, int i) { return b ? b[i] : 0.f; }
__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + expf(-x)); }

__device__ __forceinline__ int32_t prev_token(const ChainArgs& a, int p, int b) {
  int32_t t = p == 0 ? a.t0[b]
                     : amax_index(__hip_atomic_load(&a.keys[(size_t)(p - 1) * a.B + b], __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT));
  return (t < 0 || t >= a.V) ? 0 : t;  // out-of-range first tokens are flagged by chain_prologue
}

// ---- GRU weight slice resident in LDS ----------------------------------------------
// The 12 weight rows a work item needs (gates r, z, n of its 4 units) from
// W_ih and from W_hh, rows ordered (gate, unit), each padded by 8 elements so
// the 16 rows read by one MFMA fragment load fall in distinct LDS banks.
template <class W>
__device__ __forceinline__ void copy8(W* dst, const W* src) {
  if constexpr (sizeof(W) == 2) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  } else {
    reinterpret_cast<float4*>(dst)[0] = reinterpret_cast<const float4*>(src)[0];
    reinterpret_cast<float4*>(dst)[1] = reinterpret_cast<const float4*>(src)[1];
  }
}

__host__ __device__ inline size_t gru_slice_elems(int d, int Hs) { return (size_t)12 * (d + 8) + (size_t)12 * (Hs + 8); }

template <class W>
__device__ void stage_gru_slice(const ChainArgs& a, int item, W* lds) {
  const int d = a.d, Hs = a.Hs, j0 = item * 4;
  const int nx = d / 8, nh = Hs / 8;
  for (int i = threadIdx.x; i < 12 * nx; i += blockDim.x) {
    const int row = i / nx, c = i - row * nx, g = row >> 2, u = row & 3;
    copy8(lds + (size_t)row * (d + 8) + c * 8, (const W*)a.w_ih + ((size_t)g * Hs + j0 + u) * d + c * 8);
  }
  W* lh = lds + (size_t)12 * (d + 8);
  for (int i = threadIdx.x; i < 12 * nh; i += blockDim.x) {
    const int row = i / nh, c = i - row * nh, g = row >> 2, u = row & 3;
    copy8(lh + (size_t)row * (Hs + 8) + c * 8, (const W*)a.w_hh + ((size_t)g * Hs + j0 + u) * Hs + c * 8);
  }
  __syncthreads();
}

// ---- phase G: one GRU step for 4 units and all sequences ------------------------
// Left-operand row `row` = 4u + g of a work item: g = 0 r, 1 z, 2 n (input
// half only), 3 n (hidden half only), so one 16x16 result tile holds all the
// pre-activations the gates need.  The hidden half W_hh h depends only on the
// previous state and is computed ahead of the token (gru_hidden_part); the
// input half W_ih E[token] and the gates follow once the token is known.
template <class W, bool kLds>
__device__ __forceinline__ void gru_rows(const ChainArgs& a, int item, const W* lds, const W*& rx, const W*& rh,
                                         bool& has_x, bool& has_h) {
  const int lane = threadIdx.x & 63, row = lane & 15, kg = lane >> 4;
  const int d = a.d, Hs = a.Hs, j0 = item * 4;
  const int u = row >> 2, g = row & 3;
  has_x = g != 3;
  has_h = g != 2;
  const int gx = g < 3 ? g : 2, gh = g < 2 ? g : 2;
  if constexpr (kLds) {
    rx = lds + (size_t)(gx * 4 + u) * (d + 8) + kg * 8;
    rh = lds + (size_t)12 * (d + 8) + (size_t)(gh * 4 + u) * (Hs + 8) + kg * 8;
  } else {
    rx = (const W*)a.w_ih + ((size_t)gx * Hs + j0 + u) * d + kg * 8;
    rh = (const W*)a.w_hh + ((size_t)gh * Hs + j0 + u) * Hs + kg * 8;
  }
}

// MFMA right operand from GRU state slot `slot`, sequence b, elements k..k+7:
// with bf16 weights the pre-split hi/lo copy, else the fp32 state
template <class W>
__device__ __forceinline__ typename act<W>::type state_frag(const ChainArgs& a, int slot, int b, int k, bool ok) {
  if constexpr (sizeof(W) == 2) {
    bf16pair f;
    const uint16_t* hi = a.hb + (size_t)slot * a.hb_step + (size_t)b * a.Hs + k;
    f.hi = load8_or_zero(hi, ok);
    f.lo = load8_or_zero(hi + (size_t)a.B * a.Hs, ok);
    return f;
  } else {
    return act_or_zero<W>(a.h + (size_t)slot * a.h_step + (size_t)b * a.Hs + k, ok);
  }
}

// per-wave partial sums of W_hh h(p) over this wave's k chunks
template <class W, int NCB, bool kLds>
__device__ void gru_hidden_part(const ChainArgs& a, int p, int item, const W* lds, f32x4 (&acc)[NCB]) {
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (p == 0) return;  // h(0) = 0
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int Hs = a.Hs, B = a.B;
  const W *rx, *rh;
  bool has_x, has_h;
  gru_rows<W, kLds>(a, item, lds, rx, rh, has_x, has_h);
  int bb[NCB];
  bool bok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int b = cb * 16 + row;
    bok[cb] = b < B;
    bb[cb] = bok[cb] ? b : 0;
  }
  constexpr int U = NCB == 1 ? 8 : 4;
  const int nch = (Hs + 31) / 32;
  for (int c0 = wv; c0 < nch; c0 += 4 * U) {  // this wave's chunks wv, wv + 4, ... in order
    frag_t<W> A[U];
    typename act<W>::type S[U][NCB];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int c = c0 + 4 * q, k = c * 32;
      const bool kok = c < nch && k + kg * 8 < Hs;
      A[q] = load8_or_zero(rh + k, kok && has_h);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) S[q][cb] = state_frag<W>(a, p, bb[cb], k + kg * 8, kok && bok[cb]);
    }
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma(A[q], S[q][cb], acc[cb]);
  }
}

template <class W, int NCB>
__device__ void gru_gates(const ChainArgs& a, int p, int item, float* red, const f32x4 (&acc)[NCB]);

// input half on top of the hidden-half partials, then the gates: h(p+1)
template <class W, int NCB, bool kLds>
__device__ void gru_finish(const ChainArgs& a, int p, int item, float* red, const W* lds, const f32x4 (&acc_h)[NCB]) {
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int d = a.d, B = a.B;
  const W *rx, *rh;
  bool has_x, has_h;
  gru_rows<W, kLds>(a, item, lds, rx, rh, has_x, has_h);

  const W* xe[NCB];
  bool bok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int b = cb * 16 + row;
    bok[cb] = b < B;
    const int tok = bok[cb] ? prev_token(a, p, b) : 0;
    xe[cb] = (const W*)a.embed + (size_t)tok * d + kg * 8;
  }
  f32x4 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = acc_h[cb];

  // E[prev] is stored exactly in W: one MFMA per chunk
  constexpr int U = NCB == 1 ? 16 : 8;
  const int ncx = (d + 31) / 32;
  for (int c0 = wv; c0 < ncx; c0 += 4 * U) {  // this wave's chunks wv, wv + 4, ... in order
    frag_t<W> A[U], X[U][NCB];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int c = c0 + 4 * q, k = c * 32;
      const bool kok = c < ncx && k + kg * 8 < d;
      A[q] = load8_or_zero(rx + k, kok && has_x);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) X[q][cb] = load8_or_zero(xe[cb] + k, kok && bok[cb]);
    }
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma(A[q], X[q][cb], acc[cb]);
  }

  gru_gates<W, NCB>(a, p, item, red, acc);
}

// sum the four waves' pre-activation partials and apply the gates: h(p+1),
// stored fp32 and, for bf16 weights, also split into bf16 hi + lo once here
// rather than by every reader
template <class W, int NCB>
__device__ void gru_gates(const ChainArgs& a, int p, int item, float* red, const f32x4 (&acc)[NCB]) {
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int Hs = a.Hs, B = a.B, j0 = item * 4;
  const float* h_in = a.h + (size_t)p * a.h_step;
  float* h_out = a.h + (size_t)(p + 1) * a.h_step;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
    *reinterpret_cast<float4*>(&red[((wv * NCB + cb) * 64 + lane) * 4]) =
        make_float4(acc[cb][0], acc[cb][1], acc[cb][2], acc[cb][3]);
  __syncthreads();
  if (wv < NCB) {
    const int cb = wv;
    float pre[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 v = *reinterpret_cast<const float4*>(&red[((w * NCB + cb) * 64 + lane) * 4]);
      pre[0] += v.x;
      pre[1] += v.y;
      pre[2] += v.z;
      pre[3] += v.w;
    }
    // result rows 4*kg + i are gate i of unit j0 + kg; column = sequence
    const int b = cb * 16 + row, j = j0 + kg;
    float hn = 0.f;
    if (b < B) {
      const float rg = sigmoidf_(pre[0] + bias_at(a.b_ih, j) + bias_at(a.b_hh, j));
      const float zg = sigmoidf_(pre[1] + bias_at(a.b_ih, Hs + j) + bias_at(a.b_hh, Hs + j));
      const float ng = tanhf(pre[2] + bias_at(a.b_ih, 2 * Hs + j) + rg * (pre[3] + bias_at(a.b_hh, 2 * Hs + j)));
      hn = (1.f - zg) * ng + zg * h_in[(size_t)b * Hs + j];
      store_agent(&h_out[(size_t)b * Hs + j], hn);
    }
    if constexpr (sizeof(W) == 2) {
      // units j0..j0+3 of sequence b sit in lanes row, row+16, row+32, row+48
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = __shfl(hn, row + 16 * q);
      if (kg == 0 && b < B) {
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hi[q] = f2bf(v[q]);
          lo[q] = f2bf(v[q] - bf2f(hi[q]));
        }
        uint16_t* dst = a.hb + (size_t)(p + 1) * a.hb_step + (size_t)b * Hs + j0;
        store_agent(reinterpret_cast<uint64_t*>(dst), (uint64_t)pack2(hi[0], hi[1]) | ((uint64_t)pack2(hi[2], hi[3]) << 32));
        store_agent(reinterpret_cast<uint64_t*>(dst + (size_t)B * Hs),
                    (uint64_t)pack2(lo[0], lo[1]) | ((uint64_t)pack2(lo[2], lo[3]) << 32));
      }
    }
  }
  __syncthreads();
}

// Phase G with W_ih read from memory (kernels that give their LDS to W2).
// This wave's W_ih fragments (k chunks wv + 4j) do not depend on the token,
// so they are fetched while the workgroup still waits for it; each workgroup
// reads the same rows every step, so they stay in its XCD's L2.
constexpr int kXPre = 20;  // chunks per wave fetched ahead: all of them for d <= 2560
template <class W>
__device__ __forceinline__ void gru_x_prefetch(const ChainArgs& a, int item, frag_t<W> (&xw)[kXPre]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, kg = lane >> 4;
  const W *rx, *rh;
  bool has_x, has_h;
  gru_rows<W, false>(a, item, nullptr, rx, rh, has_x, has_h);
  const int ncx = (a.d + 31) / 32;
#pragma unroll
  for (int j = 0; j < kXPre; ++j) {
    const int c = wv + 4 * j, k = c * 32;
    xw[j] = load8_or_zero(rx + k, has_x && c < ncx && k + kg * 8 < a.d);
  }
}

template <class W, int NCB>
__device__ __forceinline__ void gru_finish_pre(const ChainArgs& a, int p, int item, float* red, const frag_t<W> (&xw)[kXPre],
                               const f32x4 (&acc_h)[NCB]) {
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int d = a.d, B = a.B;
  const W *rx, *rh;
  bool has_x, has_h;
  gru_rows<W, false>(a, item, nullptr, rx, rh, has_x, has_h);
  const W* xe[NCB];
  bool bok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int b = cb * 16 + row;
    bok[cb] = b < B;
    const int tok = bok[cb] ? prev_token(a, p, b) : 0;
    xe[cb] = (const W*)a.embed + (size_t)tok * d + kg * 8;
  }
  f32x4 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = acc_h[cb];
  const int ncx = (d + 31) / 32;
  {
    frag_t<W> X[kXPre][NCB];
#pragma unroll
    for (int j = 0; j < kXPre; ++j) {
      const int c = wv + 4 * j, k = c * 32;
      const bool kok = c < ncx && k + kg * 8 < d;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) X[j][cb] = load8_or_zero(xe[cb] + k, kok && bok[cb]);
    }
#pragma unroll
    for (int j = 0; j < kXPre; ++j)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma(xw[j], X[j][cb], acc[cb]);
  }
  // chunks beyond the prefetched ones (d > 4 * 32 * kXPre), same order, four per batch
  for (int c0 = wv + 4 * kXPre; c0 < ncx; c0 += 16) {
    frag_t<W> A[4], X[4][NCB];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + 4 * q, k = c * 32;
      const bool kok = c < ncx && k + kg * 8 < d;
      A[q] = load8_or_zero(rx + k, kok && has_x);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) X[q][cb] = load8_or_zero(xe[cb] + k, kok && bok[cb]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma(A[q], X[q][cb], acc[cb]);
  }
  DH_STAMP(p, 8);
  gru_gates<W, NCB>(a, p, item, red, acc);
}

// ---- phase W: 16 bottleneck units, all sequences ----------------------------------
// The state half of W1 for a work item, 16 rows padded by 8, resident in LDS.
template <class W>
__device__ void stage_w1_slice(const ChainArgs& a, int item, W* lds) {
  const int Hs = a.Hs, nh = Hs / 8, k0 = item * 16;
  for (int i = threadIdx.x; i < 16 * nh; i += blockDim.x) {
    const int row = i / nh, c = i - row * nh;
    copy8(lds + (size_t)row * (Hs + 8) + c * 8,
          (const W*)a.w1 + (size_t)min(k0 + row, a.r - 1) * (a.d + Hs) + a.d + c * 8);
  }
  __syncthreads();
}

// terms of the bottleneck that do not depend on the GRU state: the H half
// W1[:, :d] H_p (precomputed) and b1, for this lane's 4 rows; fetched before
// the state is ready
struct BottleneckPre {
  float4 zh, b1;
};
template <int NCB>
__device__ __forceinline__ BottleneckPre bottleneck_pre(const ChainArgs& a, int p, int item) {
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  BottleneckPre q;
  q.zh = make_float4(0.f, 0.f, 0.f, 0.f);
  q.b1 = q.zh;
  const int b = wv * 16 + row, k = item * 16 + kg * 4;
  if (wv < NCB && b < a.B && k < a.r) {  // r is a multiple of 8: k..k+3 are valid together
    q.zh = *reinterpret_cast<const float4*>(&a.zh[((size_t)b * a.P + p) * a.r + k]);
    if (a.b1) q.b1 = *reinterpret_cast<const float4*>(&a.b1[k]);
  }
  return q;
}

template <class W, int NCB, bool kLdsW>
__device__ void bottleneck_item(const ChainArgs& a, int p, int item, float* red, const W* w1_lds,
                                const BottleneckPre& pre_terms) {
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int Hs = a.Hs, B = a.B, r = a.r;
  const int k0 = item * 16;
  const W* rw;
  if constexpr (kLdsW)
    rw = w1_lds + (size_t)row * (Hs + 8) + kg * 8;
  else
    rw = (const W*)a.w1 + (size_t)min(k0 + row, r - 1) * (a.d + Hs) + a.d + kg * 8;
  int bb[NCB];
  bool bok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int b = cb * 16 + row;
    bok[cb] = b < B;
    bb[cb] = bok[cb] ? b : 0;
  }
  f32x4 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int U = NCB == 1 ? 8 : 4;
  const int nch = (Hs + 31) / 32;
  for (int c0 = wv; c0 < nch; c0 += 4 * U) {  // this wave's chunks wv, wv + 4, ... in order
    frag_t<W> A[U];
    typename act<W>::type S[U][NCB];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int c = c0 + 4 * q, k = c * 32;
      const bool kok = c < nch && k + kg * 8 < Hs;
      A[q] = load8_or_zero(rw + k, kok);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) S[q][cb] = state_frag<W>(a, p + 1, bb[cb], k + kg * 8, kok && bok[cb]);
    }
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma(A[q], S[q][cb], acc[cb]);
  }
  DH_STAMP(p, 9);
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
    *reinterpret_cast<float4*>(&red[((wv * NCB + cb) * 64 + lane) * 4]) =
        make_float4(acc[cb][0], acc[cb][1], acc[cb][2], acc[cb][3]);
  __syncthreads();
  if (wv < NCB) {
    const int cb = wv;
    float pre[4] = {pre_terms.zh.x + pre_terms.b1.x, pre_terms.zh.y + pre_terms.b1.y,
                    pre_terms.zh.z + pre_terms.b1.z, pre_terms.zh.w + pre_terms.b1.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 v = *reinterpret_cast<const float4*>(&red[((w * NCB + cb) * 64 + lane) * 4]);
      pre[0] += v.x;
      pre[1] += v.y;
      pre[2] += v.z;
      pre[3] += v.w;
    }
    const int b = cb * 16 + row, k = k0 + kg * 4;
    if (b < B && k < r) {  // r is a multiple of 8, so k..k+3 are all valid
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = pre[i] / (1.f + expf(-pre[i]));
      char* slot = (char*)a.act + (size_t)p * a.act_step;
      if constexpr (sizeof(W) == 2) {
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hi[i] = f2bf(s[i]);
          lo[i] = f2bf(s[i] - bf2f(hi[i]));
        }
        uint64_t* dst = reinterpret_cast<uint64_t*>((uint16_t*)slot + (size_t)b * r + k);
        store_agent(dst, (uint64_t)pack2(hi[0], hi[1]) | ((uint64_t)pack2(hi[2], hi[3]) << 32));
        dst = reinterpret_cast<uint64_t*>((uint16_t*)slot + (size_t)B * r + (size_t)b * r + k);
        store_agent(dst, (uint64_t)pack2(lo[0], lo[1]) | ((uint64_t)pack2(lo[2], lo[3]) << 32));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) store_agent((float*)slot + (size_t)b * r + k + i, s[i]);
      }
    }
  }
  __syncthreads();
}

// ---- phase O: W2 tiles [t_begin, t_end), base add, argmax ---------------------------
#ifndef DH_O_PREFETCH
#define DH_O_PREFETCH 2  // tiles in flight per wave beyond the one being consumed
#endif
#ifndef DH_O_EARLY
#define DH_O_EARLY 2     // of those, issued before the activations are ready
#endif
#ifndef DH_W_SHARE
#define DH_W_SHARE 3     // W2 share of a bottleneck workgroup, in eighths of the others'
#endif

// Running argmax of one lane over the logits it has seen, in increasing
// vocabulary order: the value and index of its first maximum (i < 0: none
// yet).  -0 and +0 compare equal; the packed key is formed once at the end.
struct LaneMax {
  float v;
  int32_t i;
};
__device__ __forceinline__ void lane_max(LaneMax& m, float L, int32_t idx) {
  const bool take = L > m.v || m.i < 0;
  m.v = take ? L : m.v;
  m.i = take ? idx : m.i;
}
__device__ __forceinline__ uint64_t lane_key(const LaneMax& m) { return m.i < 0 ? 0 : amax_key(m.v, (uint32_t)m.i); }

// One lane's four logits of a tile, L = (Lb + b2) + (even k chunks + odd k
// chunks), folded into its running argmax and, with kWrite, written out.
// `full` (uniform): the whole tile lies inside the vocabulary.  Both phase-O
// variants use this, so they agree to the bit.
template <bool kWrite>
__device__ __forceinline__ void tile_epilogue(const ChainArgs& a, int vv, bool full, const float (&base)[4],
                                              const f32x4 (&acc)[2], bool bok, size_t lrow, LaneMax& m) {
  const int V = a.V;
  float L[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) L[e] = base[e] + (acc[0][e] + acc[1][e]);
  if (full) {
#pragma unroll
    for (int e = 0; e < 4; ++e) lane_max(m, L[e], vv + e);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (vv + e < V) lane_max(m, L[e], vv + e);
  }
  if constexpr (kWrite) {
    if (bok) {
      float* dst = a.out_logits + lrow + vv;
      if ((V & 3) == 0 && full) {
        *reinterpret_cast<float4*>(dst) = make_float4(L[0], L[1], L[2], L[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (vv + e < V) dst[e] = L[e];
      }
    }
  }
}

// Lb + b2 for one lane's four vocabulary entries vv.. of row lrow (zeros
// past V or when !ok)
__device__ __forceinline__ void load_base4(const ChainArgs& a, size_t lrow, int vv, bool ok, float (&out)[4]) {
  const float* src = a.Lb + lrow + vv;
  if (ok && (a.V & 3) == 0 && vv + 3 < a.V) {
    const float4 q = *reinterpret_cast<const float4*>(src);
    out[0] = q.x;
    out[1] = q.y;
    out[2] = q.z;
    out[3] = q.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = (ok && vv + e < a.V) ? src[e] : 0.f;
  }
  if (a.b2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] += (ok && vv + e < a.V) ? a.b2[vv + e] : 0.f;
  }
}

// W2 tiles of workgroup `wg`: the bottleneck workgroups start phase O late,
// so they take a smaller share (DH_W_SHARE / 8 of the others').
__host__ __device__ inline void o_tile_range(int wg, int G, int nW, int T, int& t_begin, int& t_end) {
  const int64_t wsh = DH_W_SHARE, units = (int64_t)nW * wsh + (int64_t)(G - nW) * 8;
  auto start_of = [&](int w) -> int64_t {
    const int64_t u = w <= nW ? (int64_t)w * wsh : (int64_t)nW * wsh + (int64_t)(w - nW) * 8;
    return (int64_t)T * u / units;
  };
  t_begin = (int)start_of(wg);
  t_end = (int)start_of(wg + 1);
}

// Resident W2.  Of a workgroup's tiles [t_begin, t_end) the first 4*NTW live
// in registers for all P steps (wave wv owns t_begin + wv + 4i, i < NTW, as
// MFMA left operands) and the rest, at most kLdsTiles, in LDS in fragment
// order (tile j, k chunk c, lane l at 16-byte slot (j*KC + c)*64 + l, so a
// wave's fragment read is 1 KB contiguous).  Slot i of wave wv is tile
// t_begin + wv + 4i throughout.  Phase O then reads no weights from memory.
constexpr int kLdsTilesPerWave = 5;
constexpr int kLdsTiles = 4 * kLdsTilesPerWave;
template <int KC>
constexpr int resident_tiles() {  // 4 AGPRs per lane per k chunk: at most 192 of them
  return KC >= 8 ? 6 : (KC >= 4 ? 12 : 8);
}
template <class W, int KC>
constexpr bool resident_fits() {
  return sizeof(W) == 2 && KC <= 8;
}
__host__ __device__ inline size_t w2_lds_tile_bytes(int KC) { return (size_t)KC * 64 * 16; }

// Loads from clamped, in-bounds addresses (no select).  Rows past V are never
// stored; k positions past r meet zero activations, so the finite weights
// read there add exactly zero.
// (t may be -1 for a workgroup that owns no tile; such rows are never used)
template <class W>
__device__ __forceinline__ const W* w2_frag_ptr(const ChainArgs& a, int t, int row, int kg, int c) {
  const int v = min(max(t * 16 + row, 0), a.V - 1);
  return (const W*)a.w2 + (size_t)v * a.r + min(c * 32 + kg * 8, a.r - 8);
}

// The register tier is loaded straight into AGPRs (the MFMA reads its left
// operand from there), so it does not compete with the VGPRs the phases use.
// The loads are not visible to the compiler's wait-count tracking, hence the
// explicit wait for all of them; later compiler-issued waits are only ever
// stricter while these are outstanding, since loads retire in order.
template <class W, int KC, int NTW>
__device__ __forceinline__ void load_resident_w2(const ChainArgs& a, int t_begin, int t_end, frag_t<W> (&w2r)[NTW][KC]) {
  static_assert(sizeof(W) == 2, "resident W2 is bf16");
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int t = min(t_begin + wv + 4 * i, t_end - 1);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const W* ptr = w2_frag_ptr<W>(a, t, row, kg, c);
      asm volatile("global_load_dwordx4 %0, %1, off" : "=a"(w2r[i][c]) : "v"(ptr) : "memory");
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// the LDS tier: tiles t_begin + 4*NTW + j, j < n_lds
template <class W, int KC>
__device__ void stage_w2_lds(const ChainArgs& a, int t_first, int n_lds, unsigned char* lds) {
  for (int q = threadIdx.x; q < n_lds * KC * 64; q += blockDim.x) {
    const int l = q & 63, c = (q >> 6) % KC, j = q / (KC * 64);
    *reinterpret_cast<uint4*>(lds + (size_t)q * 16) =
        *reinterpret_cast<const uint4*>(w2_frag_ptr<W>(a, t_first + j, l & 15, l >> 4, c));
  }
  __syncthreads();
}

// fold this workgroup's per-lane best keys into the device-wide keys of step p
template <int NCB>
__device__ __forceinline__ void publish_best(const ChainArgs& a, int p, uint64_t (&best)[NCB], uint64_t* sbest) {
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    best[cb] = umax64(best[cb], shfl_xor_u64(best[cb], 16));
    best[cb] = umax64(best[cb], shfl_xor_u64(best[cb], 32));
    if (kg == 0) sbest[(wv * NCB + cb) * 16 + row] = best[cb];
  }
  __syncthreads();
  if (threadIdx.x < NCB * 16) {
    const int cb = threadIdx.x >> 4, rr = threadIdx.x & 15, b = cb * 16 + rr;
    uint64_t m = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) m = umax64(m, sbest[(w * NCB + cb) * 16 + rr]);
    if (b < a.B && m != 0) atomicMax((unsigned long long*)&a.keys[(size_t)p * a.B + b], (unsigned long long)m);
  }
  __syncthreads();
}

// base logits, then the correction from resident W2 tiles, then the argmax;
// same arithmetic and summation order as logits_range
template <class W, int NCB, int KC, int NTW, bool kWrite, class Ready>
__device__ __forceinline__ bool logits_resident_(const ChainArgs& a, int p, int t_begin, int t_end,
                                                 const frag_t<W> (&w2r)[NTW][KC], const unsigned char* w2_lds,
                                                 uint64_t* sbest, Ready ready) {
  constexpr int NT = NTW + kLdsTilesPerWave;  // slots below NTW: registers; then LDS
  const int lane = opaque_lane(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15, kg = lane >> 4;
  const int B = a.B, r = a.r, V = a.V, P = a.P;
  const char* act_p = (const char*)a.act + (size_t)p * a.act_step;
  auto tile_of = [&](int i) { return t_begin + wv + 4 * i; };
  size_t lrow[NCB];
  bool bok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int b = cb * 16 + row;
    bok[cb] = b < B;
    lrow[cb] = ((size_t)(bok[cb] ? b : 0) * P + p) * V;
  }
  // Lb + b2 of every owned tile: inputs, fetched before the activations exist
  float lb[NCB][NT][4];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int t = tile_of(i);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) load_base4(a, lrow[cb], t * 16 + kg * 4, t < t_end, lb[cb][i]);
  }
  if (!ready()) return false;

  uint64_t best[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    LaneMax lm{0.f, -1};
    const int b = cb * 16 + row;
    typename act<W>::type bf[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int k = c * 32 + kg * 8;
      const bool ok = bok[cb] && k < r;
      if constexpr (sizeof(W) == 2) {
        const uint16_t* hi = (const uint16_t*)act_p + (size_t)b * r + k;
        bf[c].hi = load8_or_zero(hi, ok);
        bf[c].lo = load8_or_zero(hi + (size_t)B * r, ok);
      } else {
        bf[c] = load8_or_zero((const float*)act_p + (size_t)b * r + k, ok);
      }
    }
#ifdef DH_TRACE_PHASES
    __builtin_amdgcn_s_waitcnt(0);
    if (cb == 0) DH_STAMP(p, 10);
#endif
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (tile_of(i) >= t_end) break;
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      if (i < NTW) {
#pragma unroll
        for (int c = 0; c < KC; ++c) acc[c & 1] = mma(w2r[i < NTW ? i : 0][c], bf[c], acc[c & 1]);
      } else {
        const unsigned char* src = w2_lds + ((size_t)(4 * (i - NTW) + wv) * KC * 64 + lane) * 16;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const frag_t<W> w = *reinterpret_cast<const frag_t<W>*>(src + (size_t)c * 64 * 16);
          acc[c & 1] = mma(w, bf[c], acc[c & 1]);
        }
      }
      tile_epilogue<kWrite>(a, tile_of(i) * 16 + kg * 4, (tile_of(i) + 1) * 16 <= V, lb[cb][i], acc, bok[cb], lrow[cb],
                            lm);
    }
    best[cb] = lane_key(lm);
  }
  DH_STAMP(p, 6);
  publish_best<NCB>(a, p, best, sbest);
  DH_STAMP(p, 7);
  return true;
}

template <class W, int NCB, int KC, int NTW, class Ready>
__device__ __forceinline__ bool logits_resident(const ChainArgs& a, int p, int t_begin, int t_end,
                                                const frag_t<W> (&w2r)[NTW][KC], const unsigned char* w2_lds,
                                                uint64_t* sbest, Ready ready) {
  if (a.out_logits) return logits_resident_<W, NCB, KC, NTW, true>(a, p, t_begin, t_end, w2r, w2_lds, sbest, ready);
  return logits_resident_<W, NCB, KC, NTW, false>(a, p, t_begin, t_end, w2r, w2_lds, sbest, ready);
}

template <class W, int NCB, int KC>
struct TileBuf {
  frag_t<W> w[KC];    // 16 W2 rows x all of k, MFMA left operand
  float lb[NCB][4];   // base logits of this lane's 4 rows, per column block
  float b2[4];
};

// `ready` is called by the whole workgroup after the first tiles are in flight
// and before the activations are read; it returns false when the kernel must stop.
template <class W, int NCB, int KC, bool kWrite, class Ready>
__device__ __forceinline__ bool logits_range_(const ChainArgs& a, int p, int t_begin, int t_end, uint64_t* sbest,
                                              Ready ready) {
  constexpr int PF = DH_O_PREFETCH;
  const int lane = opaque_lane(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15, kg = lane >> 4;
  const int B = a.B, r = a.r, V = a.V, P = a.P;
  const bool vec4 = (V & 3) == 0;

  const char* act_p = (const char*)a.act + (size_t)p * a.act_step;
  typename act<W>::type bf[NCB][KC];
  size_t lrow[NCB];
  bool bok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int b = cb * 16 + row;
    bok[cb] = b < B;
    lrow[cb] = ((size_t)(bok[cb] ? b : 0) * P + p) * V;
  }

  LaneMax lm[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) lm[cb] = LaneMax{0.f, -1};

  const W* w2 = (const W*)a.w2;
  auto issue = [&](int t, TileBuf<W, NCB, KC>& tb) {
    if (t >= t_end) return;
    const W* wr = w2 + (size_t)min(t * 16 + row, V - 1) * r + kg * 8;
#pragma unroll
    for (int c = 0; c < KC; ++c) tb.w[c] = load8_or_zero(wr + c * 32, c * 32 + kg * 8 < r);
    const int vv = t * 16 + kg * 4;  // this lane's 4 vocabulary rows
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const float* src = a.Lb + lrow[cb] + vv;
      if (vec4 && vv + 3 < V) {
        const float4 q = *reinterpret_cast<const float4*>(src);
        tb.lb[cb][0] = q.x;
        tb.lb[cb][1] = q.y;
        tb.lb[cb][2] = q.z;
        tb.lb[cb][3] = q.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) tb.lb[cb][i] = vv + i < V ? src[i] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) tb.b2[i] = (a.b2 && vv + i < V) ? a.b2[vv + i] : 0.f;
  };

  // first tiles go out before the activations exist
  TileBuf<W, NCB, KC> ring[PF + 1];
  int t = t_begin + wv;
#pragma unroll
  for (int i = 0; i < DH_O_EARLY; ++i) issue(t + 4 * i, ring[i]);
  if (!ready()) return false;
#pragma unroll
  for (int i = DH_O_EARLY; i < PF; ++i) issue(t + 4 * i, ring[i]);

  // right operands: the bottleneck activations of every sequence, all of k
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int b = cb * 16 + row;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int k = c * 32 + kg * 8;
      const bool ok = bok[cb] && k < r;
      if constexpr (sizeof(W) == 2) {
        const uint16_t* hi = (const uint16_t*)act_p + (size_t)b * r + k;
        bf[cb][c].hi = load8_or_zero(hi, ok);
        bf[cb][c].lo = load8_or_zero(hi + (size_t)B * r, ok);
      } else {
        bf[cb][c] = load8_or_zero((const float*)act_p + (size_t)b * r + k, ok);
      }
    }
  }

  auto consume = [&](int t, const TileBuf<W, NCB, KC>& tb) {
    const int vv = t * 16 + kg * 4;
    f32x4 acc[NCB][2];  // even and odd k chunks: two independent MFMA chains
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb][0] = acc[cb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb][c & 1] = mma(tb.w[c], bf[cb][c], acc[cb][c & 1]);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float base[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) base[e] = a.b2 ? tb.lb[cb][e] + tb.b2[e] : tb.lb[cb][e];
      tile_epilogue<kWrite>(a, vv, (t + 1) * 16 <= V, base, acc[cb], bok[cb], lrow[cb], lm[cb]);
    }
  };

  // ring of PF + 1 tile buffers; slot indices are compile-time after unrolling
  while (t < t_end) {
#pragma unroll
    for (int s = 0; s < PF + 1; ++s) {
      issue(t + 4 * PF, ring[(s + PF) % (PF + 1)]);
      if (t < t_end) consume(t, ring[s]);
      t += 4;
    }
  }

  uint64_t best[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) best[cb] = lane_key(lm[cb]);
  publish_best<NCB>(a, p, best, sbest);
  return true;
}

template <class W, int NCB, int KC, class Ready>
__device__ __forceinline__ bool logits_range(const ChainArgs& a, int p, int t_begin, int t_end, uint64_t* sbest,
                                             Ready ready) {
  if (a.out_logits) return logits_range_<W, NCB, KC, true>(a, p, t_begin, t_end, sbest, ready);
  return logits_range_<W, NCB, KC, false>(a, p, t_begin, t_end, sbest, ready);
}

// ---- kernels ------------------------------------------------------------------------
// Before the steps: the H half of the bottleneck for every position,
// zh[b][p][k] = sum_i H[b][p][i] W1[k][i] (one 16x16 tile per workgroup, k
// split over the waves), and the zeroed keys, counters and initial state.
template <class W>
__global__ __launch_bounds__(256) void chain_prologue(ChainArgs a, const void* H, int reset_status) {
  __shared__ __attribute__((aligned(16))) float red[4 * 64 * 4];
  const int M = a.B * a.P;
  splitk_tile<W>((const W*)H, a.d, (const W*)a.w1, a.d + a.Hs, (float*)a.zh, a.r, M, a.r, a.d, blockIdx.x, blockIdx.y,
                 red);
  const int nblk = gridDim.x * gridDim.y, blk = blockIdx.y * gridDim.x + blockIdx.x;
  const int tid = blk * blockDim.x + threadIdx.x, stride = nblk * blockDim.x;
  for (int i = tid; i < a.P * a.B; i += stride) a.keys[i] = 0;
  for (int i = tid; i < a.B * a.Hs; i += stride) a.h[i] = 0.f;  // state slot 0
  for (int i = tid; i < 4 * kSubCounters * kCounterStride; i += stride) a.counters[i] = 0;
  if (tid == 0) {
    int32_t s = reset_status ? 0 : *a.status;
    for (int b = 0; b < a.B; ++b)
      if ((a.t0[b] < 0 || a.t0[b] >= a.V) && s == 0) s = 1;
    *a.status = s;
  }
}

// drafted tokens of step p from the packed argmax keys
__device__ __forceinline__ void write_tokens(const ChainArgs& a, int p) {
  for (int b = threadIdx.x; b < a.B; b += blockDim.x)
    a.out_tokens[(size_t)b * a.P + p] =
        amax_index(__hip_atomic_load(&a.keys[(size_t)p * a.B + b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

__global__ void chain_finalize(ChainArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < a.B * a.P) {
    const int b = i / a.P, p = i % a.P;
    a.out_tokens[i] = amax_index(a.keys[(size_t)p * a.B + b]);
  }
}

template <class W, int NCB>
__global__ __launch_bounds__(256) void chain_gru_k(ChainArgs a, int p) {
  __shared__ __attribute__((aligned(16))) float red[4 * NCB * 64 * 4];
  for (int it = blockIdx.x; it < a.Hs / 4; it += gridDim.x) {
    f32x4 acc_h[NCB];
    gru_hidden_part<W, NCB, false>(a, p, it, nullptr, acc_h);
    gru_finish<W, NCB, false>(a, p, it, red, nullptr, acc_h);
  }
}

template <class W, int NCB>
__global__ __launch_bounds__(256) void chain_bottleneck_k(ChainArgs a, int p) {
  __shared__ __attribute__((aligned(16))) float red[4 * NCB * 64 * 4];
  for (int it = blockIdx.x; it < (a.r + 15) / 16; it += gridDim.x)
    bottleneck_item<W, NCB, false>(a, p, it, red, nullptr, bottleneck_pre<NCB>(a, p, it));
}

template <class W, int NCB, int KC>
__global__ __launch_bounds__(256) void chain_logits_k(ChainArgs a, int p) {
  __shared__ uint64_t sbest[4 * NCB * 16];
  const int T = (a.V + 15) / 16, G = gridDim.x, w = blockIdx.x;
  logits_range<W, NCB, KC>(a, p, (int)((int64_t)T * w / G), (int)((int64_t)T * (w + 1) / G), sbest,
                           [] { return true; });
}

// All P steps in one cooperative launch; every workgroup owns one GRU work
// item (Hs/4 <= grid).  NTW == 0 (W2 streamed every step), kLds: 0 weights
// from global memory, 1 the GRU slice in LDS, 2 also the bottleneck slice of
// W1 in LDS.  NTW > 0 (W2 resident on chip): the GRU weights come from
// memory, W_ih fetched ahead of the token; kLds 2 puts the W1 slice in LDS;
// the LDS tier of W2 follows it.
template <class W, int NCB, int KC, int kLds, int NTW>
__global__ __launch_bounds__(256) void chain_persistent(ChainArgs a) {
  constexpr bool kGruLds = kLds >= 1 && NTW == 0;
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
  __shared__ __attribute__((aligned(16))) float red[4 * NCB * 64 * 4];
  __shared__ uint64_t sbest[4 * NCB * 16];
  W* gl = reinterpret_cast<W*>(dyn_lds);
  W* wl = gl + (kGruLds ? gru_slice_elems(a.d, a.Hs) : 0);
  const int G = gridDim.x, wg = blockIdx.x;
  const int nG = a.Hs / 4, nW = (a.r + 15) / 16, T = (a.V + 15) / 16;
  uint32_t* cG = a.counters + 0 * kSubCounters * kCounterStride;
  uint32_t* cW = a.counters + 1 * kSubCounters * kCounterStride;
  uint32_t* cO = a.counters + 2 * kSubCounters * kCounterStride;
  int t_begin, t_end;
  o_tile_range(wg, G, nW, T, t_begin, t_end);
  frag_t<W> w2r[NTW > 0 ? NTW : 1][KC];
  // LDS tier of resident W2: after the GRU slice, and after the W1 slice in
  // bottleneck workgroups
  unsigned char* w2l = reinterpret_cast<unsigned char*>(wl) +
                       (kLds >= 2 && wg < nW ? (size_t)16 * (a.Hs + 8) * sizeof(W) : 0);
  if constexpr (NTW > 0) load_resident_w2<W, KC>(a, t_begin, t_end, w2r);
  if (kGruLds && wg < nG) stage_gru_slice<W>(a, wg, gl);
  if (kLds >= 2 && wg < nW) stage_w1_slice<W>(a, wg, wl);
  if constexpr (NTW > 0) stage_w2_lds<W, KC>(a, t_begin + 4 * NTW, max(0, t_end - t_begin - 4 * NTW), w2l);
  f32x4 acc_h[NCB];  // hidden half of this workgroup's next GRU step
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc_h[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < a.P; ++p) {
    if (wg < nG) {
      if constexpr (NTW > 0) {
        frag_t<W> xw[kXPre];
        gru_x_prefetch<W>(a, wg, xw);
        if (p > 0 && !wg_wait_geq(cO, (uint32_t)(p * G), a.status)) return;
        DH_STAMP(p, 0);
        if (wg == 0 && p > 0) write_tokens(a, p - 1);
        gru_finish_pre<W, NCB>(a, p, wg, red, xw, acc_h);
      } else {
        if (p > 0 && !wg_wait_geq(cO, (uint32_t)(p * G), a.status)) return;
        DH_STAMP(p, 0);
        if (wg == 0 && p > 0) write_tokens(a, p - 1);
        gru_finish<W, NCB, kGruLds>(a, p, wg, red, gl, acc_h);
      }
    }
    wg_arrive(cG);
    DH_STAMP(p, 1);
    if (wg < nW) {
      const BottleneckPre pre = bottleneck_pre<NCB>(a, p, wg);
      if (!wg_wait_geq(cG, (uint32_t)((p + 1) * G), a.status)) return;
      DH_STAMP(p, 2);
      bottleneck_item<W, NCB, (kLds >= 2)>(a, p, wg, red, wl, pre);
    }
    wg_arrive(cW);
    DH_STAMP(p, 3);
    if (wg < nG && p + 1 < a.P) {  // W_hh h(p+1) while the bottleneck runs
      if (!wg_wait_geq(cG, (uint32_t)((p + 1) * G), a.status)) return;
      gru_hidden_part<W, NCB, kGruLds>(a, p + 1, wg, gl, acc_h);
    }
    auto ready = [&] {
      const bool ok = wg_wait_geq(cW, (uint32_t)((p + 1) * G), a.status);
      DH_STAMP(p, 4);
      return ok;
    };
    bool go;
    if constexpr (NTW > 0)
      go = logits_resident<W, NCB, KC, NTW>(a, p, t_begin, t_end, w2r, w2l, sbest, ready);
    else
      go = logits_range<W, NCB, KC>(a, p, t_begin, t_end, sbest, ready);
    if (!go) return;
    wg_arrive(cO);
    DH_STAMP(p, 5);
  }
  if (wg == 0 && wg_wait_geq(cO, (uint32_t)(a.P * G), a.status)) write_tokens(a, a.P - 1);
}

// ---- host side ------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

ChainLayout chain_layout(int d, int Hs, int r, int P, int group) {
  (void)d;
  ChainLayout L;
  size_t off = 0;
  L.status = off;
  off += 256;
  L.counters = off;
  off += (size_t)4 * kSubCounters * kCounterStride * 4;
  L.keys = off;
  off += align256((size_t)P * group * 8);
  L.zh = off;
  off += align256((size_t)group * P * r * 4);
  // one slot per step for every value handed between workgroups, so no slot
  // is read before it is written within a launch
  L.h_step = (int)(align256((size_t)group * Hs * 4) / 4);
  L.h = off;
  off += (size_t)(P + 1) * L.h_step * 4;
  L.hb_step = (int)(align256((size_t)group * Hs * 2 * 2) / 2);
  L.hb = off;
  off += (size_t)(P + 1) * L.hb_step * 2;
  L.act_step = (int)align256((size_t)group * r * 4);
  L.act = off;
  off += (size_t)P * L.act_step;
  L.trace = off;
#ifdef DH_TRACE_PHASES
  off += (size_t)P * 1024 * kTraceSlots * 8;
#endif
  L.total = off;
  return L;
}

// Dynamic LDS a resident-W2 launch on G workgroups needs (the W1 slice
// region, then the LDS tiles), or 0 if some workgroup owns more tiles than
// its register and LDS slots hold.
static size_t resident_lds(int G, const ChainArgs& a, int ntw, int kc, size_t w1_bytes) {
  const int nW = (a.r + 15) / 16, T = (a.V + 15) / 16;
  size_t need = w1_bytes;
  for (int w = 0; w < G; ++w) {
    int b, e;
    o_tile_range(w, G, nW, T, b, e);
    const int n_lds = e - b - 4 * ntw;
    if (n_lds > kLdsTiles) return 0;
    if (n_lds > 0) {
      const size_t at = (w < nW ? w1_bytes : 0) + (size_t)n_lds * w2_lds_tile_bytes(kc);
      need = at > need ? at : need;
    }
  }
  return need;
}

struct CoopGrid {
  const void* fn = nullptr;
  int device = -1;
  size_t lds = 0;
  int blocks = 0;
};

template <class W, int NCB, int KC, int kLds, int NTW>
static hipError_t launch_persistent(const ChainArgs& a, size_t lds_bytes, hipStream_t s) {
  static thread_local CoopGrid cache;
  const void* fn = (const void*)chain_persistent<W, NCB, KC, kLds, NTW>;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (cache.fn != fn || cache.device != dev || cache.lds != lds_bytes) {
    if (lds_bytes > 0) {
      e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
      if (e != hipSuccess) return e;
    }
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, lds_bytes);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    cache.fn = fn;
    cache.device = dev;
    cache.lds = lds_bytes;
    // resident W2 was sized for one workgroup per CU
    cache.blocks = NTW > 0 ? cus : cus * (per_cu > 2 ? 2 : per_cu);
  }
  if (cache.blocks < a.Hs / 4) return hipErrorInvalidConfiguration;  // one GRU item per workgroup
  ChainArgs arg = a;
  void* params[] = {&arg};
  return hipLaunchCooperativeKernel(fn, dim3(cache.blocks), dim3(256), params, (unsigned)lds_bytes, s);
}

constexpr size_t kLdsBudget = 144 * 1024;  // dynamic LDS the persistent kernel may use (160 KB per CU)

template <class W, int NCB, int KC>
static hipError_t run_chain(const ChainArgs& a, int mode, hipStream_t s, bool& persistent) {
  const int cus = device_cus();
  // the persistent schedule needs one GRU work item per workgroup
  persistent = mode != 1 && cus > 0 && a.Hs / 4 <= cus;
  if (persistent) {
    const size_t g = gru_slice_elems(a.d, a.Hs) * sizeof(W);
    const size_t w = (size_t)16 * (a.Hs + 8) * sizeof(W);
    // W2 stays on chip (registers + LDS) when every workgroup's share fits;
    // the grid is then one workgroup per CU
    if constexpr (NCB == 1 && resident_fits<W, KC>()) {
      constexpr int NTW = resident_tiles<KC>();
      if (mode == 0) {
        const size_t l2 = resident_lds(cus, a, NTW, KC, w);
        if (l2 > 0 && l2 <= kLdsBudget) return launch_persistent<W, NCB, KC, 2, NTW>(a, l2, s);
      }
    }
    if (g + w <= kLdsBudget) return launch_persistent<W, NCB, KC, 2, 0>(a, g + w, s);
    if (g <= kLdsBudget) return launch_persistent<W, NCB, KC, 1, 0>(a, g, s);
    return launch_persistent<W, NCB, KC, 0, 0>(a, 0, s);
  }
  const int nG = a.Hs / 4, nW = (a.r + 15) / 16, T = (a.V + 15) / 16;
  const int nO = T < cus ? T : (cus > 0 ? cus : 256);
  for (int p = 0; p < a.P; ++p) {
    hipLaunchKernelGGL((chain_gru_k<W, NCB>), dim3(nG), dim3(256), 0, s, a, p);
    hipLaunchKernelGGL((chain_bottleneck_k<W, NCB>), dim3(nW), dim3(256), 0, s, a, p);
    hipLaunchKernelGGL((chain_logits_k<W, NCB, KC>), dim3(nO), dim3(256), 0, s, a, p);
  }
  return hipGetLastError();
}

// k chunks of 32 in the bottleneck, rounded up to 1, 2, 4 or 8 (zero padded)
template <class W, int NCB>
static hipError_t run_chain_kc(const ChainArgs& a, int mode, hipStream_t s, bool& persistent) {
  const int kc = (a.r + 31) / 32;
  if (kc <= 1) return run_chain<W, NCB, 1>(a, mode, s, persistent);
  if (kc <= 2) return run_chain<W, NCB, 2>(a, mode, s, persistent);
  if (kc <= 4) return run_chain<W, NCB, 4>(a, mode, s, persistent);
  if (kc <= 8) return run_chain<W, NCB, 8>(a, mode, s, persistent);
  return hipErrorInvalidValue;
}

hipError_t launch_chain(int dtype, const ChainArgs& a, const void* H, int mode, bool reset_status, hipStream_t s,
                        hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (a.B <= 0) return hipSuccess;
  const dim3 pro((a.r + 15) / 16, (a.B * a.P + 15) / 16);
  if (dtype == kBF16)
    hipLaunchKernelGGL(chain_prologue<uint16_t>, pro, dim3(256), 0, s, a, H, reset_status ? 1 : 0);
  else
    hipLaunchKernelGGL(chain_prologue<float>, pro, dim3(256), 0, s, a, H, reset_status ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool two = a.B > 16;
  bool persistent = false;
  if (ev_start && ev_stop) {
    e = hipEventRecord(ev_start, s);
    if (e != hipSuccess) return e;
  }
  if (dtype == kBF16)
    e = two ? run_chain_kc<uint16_t, 2>(a, mode, s, persistent) : run_chain_kc<uint16_t, 1>(a, mode, s, persistent);
  else
    e = two ? run_chain_kc<float, 2>(a, mode, s, persistent) : run_chain_kc<float, 1>(a, mode, s, persistent);
  if (e != hipSuccess) return e;
  if (ev_start && ev_stop) {
    e = hipEventRecord(ev_stop, s);
    if (e != hipSuccess) return e;
  }
  if (!persistent) hipLaunchKernelGGL(chain_finalize, dim3((a.B * a.P + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dh
