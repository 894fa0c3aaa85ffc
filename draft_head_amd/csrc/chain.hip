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
#ifdef DH_TRACE_PHASES
#define DH_STAMP(p, slot) \
  do { if (a.trace && threadIdx.x == 0) a.trace[((size_t)(p) * gridDim.x + blockIdx.x) * 6 + (slot)] = wall_clock64(); } while (0)
#else
#define DH_STAMP(p, slot) \
  do { } while (0)
#endif

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

// per-wave partial sums of W_hh h(p) over this wave's k chunks
template <class W, int NCB, bool kLds>
__device__ void gru_hidden_part(const ChainArgs& a, int p, int item, const W* lds, f32x4 (&acc)[NCB]) {
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (p == 0) return;  // h(0) = 0
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int Hs = a.Hs, B = a.B;
  const W *rx, *rh;
  bool has_x, has_h;
  gru_rows<W, kLds>(a, item, lds, rx, rh, has_x, has_h);
  const float* h_in = a.h + (size_t)p * a.h_step;
  const float* hv[NCB];
  bool bok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int b = cb * 16 + row;
    bok[cb] = b < B;
    hv[cb] = h_in + (size_t)(bok[cb] ? b : 0) * Hs + kg * 8;
  }
  constexpr int U = NCB == 1 ? 8 : 4;
  const int nch = (Hs + 31) / 32;
  for (int c0 = wv * U; c0 < nch; c0 += 4 * U) {
    frag_t<W> A[U];
    typename act<W>::type S[U][NCB];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int k = (c0 + q) * 32;
      const bool kok = c0 + q < nch && k + kg * 8 < Hs;
      A[q] = load8_or_zero(rh + k, kok && has_h);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) S[q][cb] = act_or_zero<W>(hv[cb] + k, kok && bok[cb]);
    }
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma(A[q], S[q][cb], acc[cb]);
  }
}

// input half on top of the hidden-half partials, then the gates: h(p+1)
template <class W, int NCB, bool kLds>
__device__ void gru_finish(const ChainArgs& a, int p, int item, float* red, const W* lds, const f32x4 (&acc_h)[NCB]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int d = a.d, Hs = a.Hs, B = a.B;
  const int j0 = item * 4;
  const W *rx, *rh;
  bool has_x, has_h;
  gru_rows<W, kLds>(a, item, lds, rx, rh, has_x, has_h);
  const float* h_in = a.h + (size_t)p * a.h_step;
  float* h_out = a.h + (size_t)(p + 1) * a.h_step;

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
  for (int c0 = wv * U; c0 < ncx; c0 += 4 * U) {
    frag_t<W> A[U], X[U][NCB];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int k = (c0 + q) * 32;
      const bool kok = c0 + q < ncx && k + kg * 8 < d;
      A[q] = load8_or_zero(rx + k, kok && has_x);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) X[q][cb] = load8_or_zero(xe[cb] + k, kok && bok[cb]);
    }
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma(A[q], X[q][cb], acc[cb]);
  }

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
    if (b < B) {
      const float rg = sigmoidf_(pre[0] + bias_at(a.b_ih, j) + bias_at(a.b_hh, j));
      const float zg = sigmoidf_(pre[1] + bias_at(a.b_ih, Hs + j) + bias_at(a.b_hh, Hs + j));
      const float ng = tanhf(pre[2] + bias_at(a.b_ih, 2 * Hs + j) + rg * (pre[3] + bias_at(a.b_hh, 2 * Hs + j)));
      store_agent(&h_out[(size_t)b * Hs + j], (1.f - zg) * ng + zg * h_in[(size_t)b * Hs + j]);
    }
  }
  __syncthreads();
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
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
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
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int Hs = a.Hs, B = a.B, r = a.r;
  const int k0 = item * 16;
  const W* rw;
  if constexpr (kLdsW)
    rw = w1_lds + (size_t)row * (Hs + 8) + kg * 8;
  else
    rw = (const W*)a.w1 + (size_t)min(k0 + row, r - 1) * (a.d + Hs) + a.d + kg * 8;
  const float* h_new = a.h + (size_t)(p + 1) * a.h_step;
  const float* hv[NCB];
  bool bok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int b = cb * 16 + row;
    bok[cb] = b < B;
    hv[cb] = h_new + (size_t)(bok[cb] ? b : 0) * Hs + kg * 8;
  }
  f32x4 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int U = NCB == 1 ? 8 : 4;
  const int nch = (Hs + 31) / 32;
  for (int c0 = wv * U; c0 < nch; c0 += 4 * U) {
    frag_t<W> A[U];
    typename act<W>::type S[U][NCB];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int k = (c0 + q) * 32;
      const bool kok = c0 + q < nch && k + kg * 8 < Hs;
      A[q] = load8_or_zero(rw + k, kok);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) S[q][cb] = act_or_zero<W>(hv[cb] + k, kok && bok[cb]);
    }
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma(A[q], S[q][cb], acc[cb]);
  }
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

template <class W, int NCB, int KC>
struct TileBuf {
  frag_t<W> w[KC];    // 16 W2 rows x all of k, MFMA left operand
  float lb[NCB][4];   // base logits of this lane's 4 rows, per column block
  float b2[4];
};

// `ready` is called by the whole workgroup after the first tiles are in flight
// and before the activations are read; it returns false when the kernel must stop.
template <class W, int NCB, int KC, class Ready>
__device__ bool logits_range(const ChainArgs& a, int p, int t_begin, int t_end, uint64_t* sbest, Ready ready) {
  constexpr int PF = DH_O_PREFETCH;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
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

  uint64_t best[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) best[cb] = 0;

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
      if (!bok[cb]) continue;
      float L[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        L[i] = tb.lb[cb][i] + (acc[cb][0][i] + acc[cb][1][i]) + tb.b2[i];
        if (vv + i < V) best[cb] = umax64(best[cb], amax_key(L[i], (uint32_t)(vv + i)));
      }
      if (a.out_logits) {
        float* dst = a.out_logits + lrow[cb] + vv;
        if (vec4 && vv + 3 < V) {
          *reinterpret_cast<float4*>(dst) = make_float4(L[0], L[1], L[2], L[3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (vv + i < V) dst[i] = L[i];
        }
      }
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
    if (b < B && m != 0) atomicMax((unsigned long long*)&a.keys[(size_t)p * B + b], (unsigned long long)m);
  }
  __syncthreads();
  return true;
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
// item (Hs/4 <= grid).  kLds: 0 weights from global memory, 1 the GRU slice
// in LDS, 2 also the bottleneck slice of W1 in LDS.
template <class W, int NCB, int KC, int kLds>
__global__ __launch_bounds__(256) void chain_persistent(ChainArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
  __shared__ __attribute__((aligned(16))) float red[4 * NCB * 64 * 4];
  __shared__ uint64_t sbest[4 * NCB * 16];
  W* gl = reinterpret_cast<W*>(dyn_lds);
  W* wl = gl + (kLds >= 1 ? gru_slice_elems(a.d, a.Hs) : 0);
  const int G = gridDim.x, wg = blockIdx.x;
  const int nG = a.Hs / 4, nW = (a.r + 15) / 16, T = (a.V + 15) / 16;
  uint32_t* cG = a.counters + 0 * kSubCounters * kCounterStride;
  uint32_t* cW = a.counters + 1 * kSubCounters * kCounterStride;
  uint32_t* cO = a.counters + 2 * kSubCounters * kCounterStride;
  // W2 tiles: the bottleneck workgroups start the phase late, so they take a
  // smaller share (DH_W_SHARE / 8 of the others')
  int t_begin, t_end;
  {
    const int64_t wsh = DH_W_SHARE, units = (int64_t)nW * wsh + (int64_t)(G - nW) * 8;
    auto start_of = [&](int w) -> int64_t {
      const int64_t u = w <= nW ? (int64_t)w * wsh : (int64_t)nW * wsh + (int64_t)(w - nW) * 8;
      return (int64_t)T * u / units;
    };
    t_begin = (int)start_of(wg);
    t_end = (int)start_of(wg + 1);
  }
  if (kLds >= 1 && wg < nG) stage_gru_slice<W>(a, wg, gl);
  if (kLds >= 2 && wg < nW) stage_w1_slice<W>(a, wg, wl);
  f32x4 acc_h[NCB];  // hidden half of this workgroup's next GRU step
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc_h[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < a.P; ++p) {
    if (wg < nG) {
      if (p > 0 && !wg_wait_geq(cO, (uint32_t)(p * G), a.status)) return;
      DH_STAMP(p, 0);
      if (wg == 0 && p > 0) write_tokens(a, p - 1);
      gru_finish<W, NCB, (kLds >= 1)>(a, p, wg, red, gl, acc_h);
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
      gru_hidden_part<W, NCB, (kLds >= 1)>(a, p + 1, wg, gl, acc_h);
    }
    if (!logits_range<W, NCB, KC>(a, p, t_begin, t_end, sbest, [&] {
          const bool ok = wg_wait_geq(cW, (uint32_t)((p + 1) * G), a.status);
          DH_STAMP(p, 4);
          return ok;
        }))
      return;
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
  L.act_step = (int)align256((size_t)group * r * 4);
  L.act = off;
  off += (size_t)P * L.act_step;
  L.trace = off;
#ifdef DH_TRACE_PHASES
  off += (size_t)P * 1024 * 6 * 8;
#endif
  L.total = off;
  return L;
}

struct CoopGrid {
  const void* fn = nullptr;
  int device = -1;
  size_t lds = 0;
  int blocks = 0;
};

template <class W, int NCB, int KC, int kLds>
static hipError_t launch_persistent(const ChainArgs& a, size_t lds_bytes, hipStream_t s) {
  static thread_local CoopGrid cache;
  const void* fn = (const void*)chain_persistent<W, NCB, KC, kLds>;
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
    cache.blocks = cus * (per_cu > 2 ? 2 : per_cu);
  }
  if (cache.blocks < a.Hs / 4) return hipErrorInvalidConfiguration;  // one GRU item per workgroup
  ChainArgs arg = a;
  void* params[] = {&arg};
  return hipLaunchCooperativeKernel(fn, dim3(cache.blocks), dim3(256), params, (unsigned)lds_bytes, s);
}

static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 0;
  return cus;
}

constexpr size_t kLdsBudget = 144 * 1024;  // dynamic LDS the persistent kernel may use (160 KB per CU)

template <class W, int NCB, int KC>
static hipError_t run_chain(const ChainArgs& a, int mode, hipStream_t s, bool& persistent) {
  const int cus = device_cus();
  // the persistent schedule needs one GRU work item per workgroup
  persistent = mode == 0 && cus > 0 && a.Hs / 4 <= cus;
  if (persistent) {
    const size_t g = gru_slice_elems(a.d, a.Hs) * sizeof(W);
    const size_t w = (size_t)16 * (a.Hs + 8) * sizeof(W);
    if (g + w <= kLdsBudget) return launch_persistent<W, NCB, KC, 2>(a, g + w, s);
    if (g <= kLdsBudget) return launch_persistent<W, NCB, KC, 1>(a, g, s);
    return launch_persistent<W, NCB, KC, 0>(a, 0, s);
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
