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
//   O  W2 + base add + argmax.  Each workgroup owns a contiguous range of
//      16-row W2 tiles, keeps the bottleneck fragments in registers, adds the
//      base-logit row in the MFMA epilogue and folds (value, index) into one
//      64-bit key per sequence: wave shuffles, then LDS, then one result per
//      workgroup.  Full logits are written only on request.
// The drafted token never leaves the device: phase G of the next step reduces
// the workgroups' results.
//
// Schedules that compute identical values:
//  * persistent: one launch for all P steps (all workgroups resident).  Values cross
//    workgroups as tagged hand-off words that readers poll (bounded waits);
//    W2 either stays on chip for the whole launch or is streamed every step;
//  * stepwise: three launches per step on the caller's stream, with a device
//    wide atomic max per workgroup for the argmax.
#include <mutex>

#include "device.h"
#include "internal.h"

namespace dh {

// Opt-in phase timestamps (constant 100 MHz clock) for tuning builds only.
[[maybe_unused]] constexpr int kTraceSlots = 16;
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

// an int the compiler cannot see through (keeps a loop-invariant LDS read
// inside the loop, where it costs a few registers instead of many)
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

__device__ __forceinline__ float bias_at(const float* b, int i) { return b ? b[i] : 0.f; }
__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + expf(-x)); }

__device__ __forceinline__ int32_t clamp_token(const ChainArgs& a, int32_t t) { return (t < 0 || t >= a.V) ? 0 : t; }

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

__device__ __forceinline__ void store8(uint16_t* p, const bf16x8& v) {
  *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, v);
}
__device__ __forceinline__ void store8(float* p, const f32x8& v) {
  reinterpret_cast<float4*>(p)[0] = v.lo;
  reinterpret_cast<float4*>(p)[1] = v.hi;
}

// n pieces of 8 elements, piece q from src(q) to dst(q) (LDS), with NB pieces
// per thread loaded before any of them is stored: a loop of single
// load-then-store pairs waits one memory round trip per piece.  Indices past
// the end repeat piece n - 1 (the same bytes to the same place), so no store
// sits in a branch the compiler could sink its load into.
template <class W, int NB, class Src, class Dst>
__device__ __forceinline__ void copy8_batched(int n, Src src, Dst dst) {
  if (n <= 0) return;
  for (int q0 = 0; q0 < n; q0 += NB * (int)blockDim.x) {
    typename frag<W>::type v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) v[u] = load8(src(min(q0 + u * (int)blockDim.x + (int)threadIdx.x, n - 1)));
#pragma unroll
    for (int u = 0; u < NB; ++u) store8(dst(min(q0 + u * (int)blockDim.x + (int)threadIdx.x, n - 1)), v[u]);
  }
}

template <class W>
__device__ __forceinline__ void stage_gru_slice(const ChainArgs& a, int item, W* lds) {
  const int d = a.d, Hs = a.Hs, j0 = item * 4;
  const int nx = d / 8, nh = Hs / 8;
  W* lh = lds + (size_t)12 * (d + 8);
  // W_ih rows then W_hh rows, as one list of pieces
  copy8_batched<W, 11>(
      12 * (nx + nh),
      [&](int i) -> const W* {
        if (i < 12 * nx) {
          const int row = i / nx, c = i - row * nx;
          return (const W*)a.w_ih + ((size_t)(row >> 2) * Hs + j0 + (row & 3)) * d + c * 8;
        }
        const int ih = i - 12 * nx, row = ih / nh, c = ih - row * nh;
        return (const W*)a.w_hh + ((size_t)(row >> 2) * Hs + j0 + (row & 3)) * Hs + c * 8;
      },
      [&](int i) -> W* {
        if (i < 12 * nx) {
          const int row = i / nx, c = i - row * nx;
          return lds + (size_t)row * (d + 8) + c * 8;
        }
        const int ih = i - 12 * nx, row = ih / nh, c = ih - row * nh;
        return lh + (size_t)row * (Hs + 8) + c * 8;
      });
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

// s_sleep units between polls of the waits for the state off the critical path
constexpr int kHiddenSleep = 16;

// The same right operand from a hand-off slot with n elements per row
// (bf16 weights: words [0, n/2) hold hi pairs, [n/2, n) lo pairs; fp32: one
// value per word).  Returns whether every word read carries `tag`.  (Its
// callers poll off the critical path or for many sequences; the words are
// checked as they come, which needs fewer registers than loading them all
// first.)
template <class W>
__device__ __forceinline__ bool ll_frag(const uint64_t* slot, int n, int b, int k, uint32_t tag, bool ok,
                                        typename act<W>::type& out) {
  if (!ok) {
    out = act<W>::zero();
    return true;
  }
  const uint64_t* row = slot + (size_t)b * n;
  bool good = true;
  if constexpr (sizeof(W) == 2) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t wh = ld_agent64(row + k / 2 + i), wl = ld_agent64(row + n / 2 + k / 2 + i);
      good = good & (int)ll_ok(wh, tag) & (int)ll_ok(wl, tag);
      h[i] = ll_data(wh);
      l[i] = ll_data(wl);
    }
    out.hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
    out.lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
  } else {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint64_t w = ld_agent64(row + k + i);
      good = good & ll_ok(w, tag);
      v[i] = __uint_as_float(ll_data(w));
    }
    out.lo = make_float4(v[0], v[1], v[2], v[3]);
    out.hi = make_float4(v[4], v[5], v[6], v[7]);
  }
  return good;
}

// The same right operand from hand-off words already staged in LDS as their
// data (dst[b * n + q] = word q of row b).
template <class W>
__device__ __forceinline__ typename act<W>::type staged_frag(const uint32_t* st, int n, int b, int k, bool ok) {
  if (!ok) return act<W>::zero();
  const uint32_t* row = st + (size_t)b * n;
  if constexpr (sizeof(W) == 2) {
    bf16pair f;
    f.hi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(row + k / 2));
    f.lo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(row + n / 2 + k / 2));
    return f;
  } else {
    f32x8 f;
    f.lo = *reinterpret_cast<const float4*>(row + k);
    f.hi = *reinterpret_cast<const float4*>(row + k + 4);
    return f;
  }
}

__host__ __device__ inline bool stage_state(int B, int Hs) { return B * Hs <= 8 * 256; }

// n hand-off words of `slot` carrying `tag`, polled by the whole workgroup (a
// few words per thread per round) and staged in LDS as their data.
constexpr int kStageWordsPerThread = 8;
struct IdentityIndex {
  __device__ int operator()(int q) const { return q; }
};
template <class Index = IdentityIndex>
__device__ __forceinline__ void stage_words_ll(int32_t* status, const uint64_t* slot, int n, uint32_t tag,
                                               uint32_t* dst, Index index = Index()) {
  const int bd = blockDim.x, tid = threadIdx.x;
  for (int base = 0; base < n; base += kStageWordsPerThread * bd) {
    const int ni = min(kStageWordsPerThread, (n - base + bd - 1) / bd);  // the same in every thread
    uint32_t v[kStageWordsPerThread];
    ll_wait(status, [&] {
      // every load before any tag check (a check between two loads, or a
      // load under a lane-dependent branch, waits a round trip per word);
      // lanes past the end re-read word n - 1
      uint64_t w[kStageWordsPerThread];
#pragma unroll
      for (int i = 0; i < kStageWordsPerThread; ++i)
        if (i < ni) w[i] = ld_agent64(slot + min(base + tid + i * bd, n - 1));
      bool good = true;
#pragma unroll
      for (int i = 0; i < kStageWordsPerThread; ++i)
        if (i < ni) {
          good = good & ll_ok(w[i], tag);
          v[i] = ll_data(w[i]);
        }
      return good;
    });
#pragma unroll
    for (int i = 0; i < kStageWordsPerThread; ++i) {
      const int q = base + tid + i * bd;
      if (i < ni && q < n) dst[index(q)] = v[i];
    }
  }
  __syncthreads();
}

// four consecutive values v of row b, elements k..k+3 (k a multiple of 4),
// into a hand-off slot with n elements per row, as ll_frag reads them
template <class W>
__device__ __forceinline__ void ll_put4(uint64_t* slot, int n, int b, int k, const float (&v)[4], uint32_t tag) {
  uint64_t* row = slot + (size_t)b * n;
  if constexpr (sizeof(W) == 2) {
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hi[i] = f2bf(v[i]);
      lo[i] = f2bf(v[i] - bf2f(hi[i]));
    }
    ll_put(row + k / 2, pack2(hi[0], hi[1]), tag);
    ll_put(row + k / 2 + 1, pack2(hi[2], hi[3]), tag);
    ll_put(row + n / 2 + k / 2, pack2(lo[0], lo[1]), tag);
    ll_put(row + n / 2 + k / 2 + 1, pack2(lo[2], lo[3]), tag);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) ll_put(row + k + i, __float_as_uint(v[i]), tag);
  }
}

// The GRU pre-activations are sums over k chunks of 32 in sixteen chains:
// chain v = w + 4j takes, in increasing order, the chunks c with c % 4 == w
// and (c / 4) % 4 == j, the hidden-half chunks first, then the input-half
// ones; the total is sum over w of (sum over j of chain (w, j)), both left to
// right.  A kernel with four waves keeps chains (w, 0..3) in wave w; one with
// sixteen keeps chain v in wave v; they produce the same bits.
constexpr int kGruChains = 16;

// per-wave partial sums of W_hh h(p) over this wave's k chunks, chains (wv, 0..3)
// kLL: the state comes as hand-off words of the persistent launch `ep`
// seq0: first sequence of this work item's 16 NCB columns (three-launch schedule)
template <class W, int NCB, bool kLds, bool kLL = false>
__device__ __forceinline__ void gru_hidden_part(const ChainArgs& a, int p, int item, const W* lds, f32x4 (&acc)[4][NCB], uint32_t ep = 0,
                                                int seq0 = 0) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[j][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
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
    const int b = seq0 + cb * 16 + row;
    bok[cb] = b < B;
    bb[cb] = bok[cb] ? b : 0;
  }
  constexpr int U = NCB == 1 ? 8 : 4;  // a multiple of 4: chunk c0 + 4q is in chain (wv, q % 4)
  const int nch = (Hs + 31) / 32;
  for (int c0 = wv; c0 < nch; c0 += 4 * U) {  // this wave's chunks wv, wv + 4, ... in order
    frag_t<W> A[U];
    typename act<W>::type S[U][NCB];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int c = c0 + 4 * q, k = c * 32;
      const bool kok = c < nch && k + kg * 8 < Hs;
      A[q] = load8_or_zero(rh + k, kok && has_h);
      if constexpr (!kLL) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) S[q][cb] = state_frag<W>(a, p, bb[cb], k + kg * 8, kok && bok[cb]);
      }
    }
    if constexpr (kLL) {  // h(p) was written at step p - 1; off the critical path, so polled gently
      const uint64_t* slot = a.ll_h + (size_t)p * B * Hs;
      ll_wait<kHiddenSleep>(a.status, [&] {
        bool good = true;
#pragma unroll
        for (int q = 0; q < U; ++q) {
          const int c = c0 + 4 * q, k = c * 32;
          const bool kok = c < nch && k + kg * 8 < Hs;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            good = ll_frag<W>(slot, Hs, bb[cb], k + kg * 8, ll_tag(ep, p - 1), kok && bok[cb], S[q][cb]) & good;
        }
        return good;
      });
    }
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[q & 3][cb] = mma(A[q], S[q][cb], acc[q & 3][cb]);
  }
}

// The input half W_ih E[prev] of this lane's unit (r, z, n gates) read from
// the per-token table (kernels instantiated with kTab), for the lanes that
// apply the gates (wave cb < NCB: sequence seq0 + 16 cb + row, unit
// 4 item + kg); zeros elsewhere.  tok: the previous tokens by sequence, or
// null to read them from the argmax keys / first tokens.
template <int NCB>
__device__ __forceinline__ float4 gru_table_in(const ChainArgs& a, int p, int item, const int32_t* tok, int seq0 = 0) {
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int b = seq0 + wv * 16 + row;
  float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
  if (wv < NCB && b < a.B) {
    const int t = tok ? clamp_token(a, tok[b]) : prev_token(a, p, b);
    const float* q = a.xt + (size_t)t * 3 * a.Hs + item * 4 + kg;
    x = make_float4(q[0], q[a.Hs], q[2 * a.Hs], 0.f);
  }
  return x;
}

template <class W, int NCB, bool kLL, bool kTab = false>
__device__ __forceinline__ void gru_gates(const ChainArgs& a, int p, int item, float* red, const f32x4 (&acc)[4][NCB], float& h_own,
                          uint32_t ep, int seq0 = 0, float4 xin = float4{0.f, 0.f, 0.f, 0.f});

// input half on top of the hidden-half partials, then the gates: h(p+1)
// tok: this step's previous tokens by sequence (raw argmax indices), or
// null to read them from the argmax keys / first tokens
template <class W, int NCB, bool kLds, bool kLL = false, bool kTab = false>
__device__ __forceinline__ void gru_finish(const ChainArgs& a, int p, int item, float* red, const W* lds, const f32x4 (&acc_h)[4][NCB],
                           const int32_t* tok = nullptr, float* h_own = nullptr, uint32_t ep = 0, int seq0 = 0) {
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
    const int b = seq0 + cb * 16 + row;
    bok[cb] = b < B;
    const int t_ = bok[cb] ? (tok ? clamp_token(a, tok[b]) : prev_token(a, p, b)) : 0;
    xe[cb] = (const W*)a.embed + (size_t)t_ * d + kg * 8;
  }
  f32x4 acc[4][NCB];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[j][cb] = acc_h[j][cb];

  // E[prev] is stored exactly in W: one MFMA per chunk (U a multiple of 4,
  // as above).  With the per-token table the input half is read instead.
  constexpr int U = NCB == 1 ? 16 : 8;
  const int ncx = kTab ? 0 : (d + 31) / 32;
  const float4 xin = kTab ? gru_table_in<NCB>(a, p, item, tok, seq0) : float4{0.f, 0.f, 0.f, 0.f};
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
      for (int cb = 0; cb < NCB; ++cb) acc[q & 3][cb] = mma(A[q], X[q][cb], acc[q & 3][cb]);
  }

  float h_dummy = 0.f;
  gru_gates<W, NCB, kLL, kTab>(a, p, item, red, acc, h_own ? *h_own : h_dummy, ep, seq0, xin);
}

// Sum the four waves' pre-activation partials and apply the gates: h(p+1).
// Stepwise: stored fp32 and, for bf16 weights, also split into bf16 hi + lo
// once here rather than by every reader.  kLL (persistent): the lane keeps
// its own unit's fp32 state in h_own across steps, and the state goes out as
// hand-off words only.
template <class W, int NCB, bool kLL, int NWG = 4, bool kTab = false>
__device__ __forceinline__ void gru_apply(const ChainArgs& a, int p, int item, float* red, float& h_own, uint32_t ep,
                                          int seq0, float4 xin);

// four waves: each folds its own chains (wv, 0..3), then the waves' sums are added in order
template <class W, int NCB, bool kLL, bool kTab>
__device__ __forceinline__ void gru_gates(const ChainArgs& a, int p, int item, float* red, const f32x4 (&acc)[4][NCB], float& h_own,
                          uint32_t ep, int seq0, float4 xin) {
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const f32x4 s = ((acc[0][cb] + acc[1][cb]) + acc[2][cb]) + acc[3][cb];
    *reinterpret_cast<float4*>(&red[((wv * NCB + cb) * 64 + lane) * 4]) = make_float4(s[0], s[1], s[2], s[3]);
  }
  gru_apply<W, NCB, kLL, 4, kTab>(a, p, item, red, h_own, ep, seq0, xin);
}

// red holds, per wave w of NWG and column block cb, the float4 of every lane:
// NWG 4, wave w's sum of its chains; NWG 16, chain w alone.  Totals them in
// the canonical order, applies the gates and hands out h(p+1).
template <class W, int NCB, bool kLL, int NWG, bool kTab>
__device__ __forceinline__ void gru_apply(const ChainArgs& a, int p, int item, float* red, float& h_own, uint32_t ep,
                                          int seq0, float4 xin) {
  static_assert(NWG == 4 || NWG == 16, "four waves with four chains each, or one chain per wave");
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int Hs = a.Hs, B = a.B, j0 = item * 4;
  const float* h_in = a.h + (size_t)p * a.h_step;
  float* h_out = a.h + (size_t)(p + 1) * a.h_step;
  __syncthreads();
  if (wv < NCB) {
    const int cb = wv;
    auto part = [&](int w) { return *reinterpret_cast<const float4*>(&red[((w * NCB + cb) * 64 + lane) * 4]); };
    float pre[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float4 v = part(w);
      if constexpr (NWG == 16) {
#pragma unroll
        for (int j = 1; j < 4; ++j) {
          const float4 u = part(w + 4 * j);
          v = make_float4(v.x + u.x, v.y + u.y, v.z + u.z, v.w + u.w);
        }
      }
      pre[0] += v.x;
      pre[1] += v.y;
      pre[2] += v.z;
      pre[3] += v.w;
    }
    if constexpr (kTab) {  // the input half from the per-token table, after the hidden half's chains
      pre[0] += xin.x;
      pre[1] += xin.y;
      pre[2] += xin.z;
    }
    // result rows 4*kg + i are gate i of unit j0 + kg; column = sequence
    const int b = seq0 + cb * 16 + row, j = j0 + kg;
    float hn = 0.f;
    if (b < B) {
      const float rg = sigmoidf_(pre[0] + bias_at(a.b_ih, j) + bias_at(a.b_hh, j));
      const float zg = sigmoidf_(pre[1] + bias_at(a.b_ih, Hs + j) + bias_at(a.b_hh, Hs + j));
      const float ng = tanhf(pre[2] + bias_at(a.b_ih, 2 * Hs + j) + rg * (pre[3] + bias_at(a.b_hh, 2 * Hs + j)));
      if constexpr (kLL) {
        hn = (1.f - zg) * ng + zg * h_own;
        h_own = hn;
      } else {
        hn = (1.f - zg) * ng + zg * h_in[(size_t)b * Hs + j];
        store_agent(&h_out[(size_t)b * Hs + j], hn);
      }
    }
    if constexpr (kLL) {
      // units j0..j0+3 of sequence b sit in lanes row, row+16, row+32, row+48
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = __shfl(hn, row + 16 * q);
      if (kg == 0 && b < B) ll_put4<W>(a.ll_h + (size_t)(p + 1) * B * Hs, Hs, b, j0, v, ll_tag(ep, p));
    } else if constexpr (sizeof(W) == 2) {
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
constexpr int kXPre = 12;  // chunks per wave fetched ahead (the register budget allows no more)
static_assert(kXPre % 4 == 0, "chunk wv + 4j is in chain (wv, j % 4)");
constexpr int kXTail = 20;  // chunks per batch after them (d <= 5120 in one more round)
static_assert(kXTail % 4 == 0, "chunk c0 + 4q is in chain (wv, q % 4)");
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

template <class W, int NCB, bool kTab = false>
__device__ __forceinline__ void gru_finish_pre(const ChainArgs& a, int p, int item, float* red, const frag_t<W> (&xw)[kXPre],
                                               const f32x4 (&acc_h)[4][NCB], const int32_t* tok, float& h_own,
                                               uint32_t ep) {
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
    const int t_ = bok[cb] ? (tok ? clamp_token(a, tok[b]) : prev_token(a, p, b)) : 0;
    xe[cb] = (const W*)a.embed + (size_t)t_ * d + kg * 8;
  }
  f32x4 acc[4][NCB];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[j][cb] = acc_h[j][cb];
  if constexpr (kTab) {  // the input half from the per-token table (xw was not fetched)
    gru_gates<W, NCB, true, true>(a, p, item, red, acc, h_own, ep, 0, gru_table_in<NCB>(a, p, item, tok));
    return;
  }
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
      for (int cb = 0; cb < NCB; ++cb) acc[j & 3][cb] = mma(xw[j], X[j][cb], acc[j & 3][cb]);
  }
  DH_STAMP(p, 12);
  // chunks beyond the prefetched ones (d > 4 * 32 * kXPre), same order
  for (int c0 = wv + 4 * kXPre; c0 < ncx; c0 += 4 * kXTail) {
    frag_t<W> A[kXTail], X[kXTail][NCB];
#pragma unroll
    for (int q = 0; q < kXTail; ++q) {
      const int c = c0 + 4 * q, k = c * 32;
      const bool kok = c < ncx && k + kg * 8 < d;
      A[q] = load8_or_zero(rx + k, kok && has_x);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) X[q][cb] = load8_or_zero(xe[cb] + k, kok && bok[cb]);
    }
#pragma unroll
    for (int q = 0; q < kXTail; ++q)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[q & 3][cb] = mma(A[q], X[q][cb], acc[q & 3][cb]);
  }
  DH_STAMP(p, 8);
  gru_gates<W, NCB, true>(a, p, item, red, acc, h_own, ep);
}

// ---- phase W: 16 bottleneck units, all sequences ----------------------------------
// The state half of W1 for a work item, 16 rows padded by 8, resident in LDS.
template <class W>
__device__ __forceinline__ void stage_w1_slice(const ChainArgs& a, int item, W* lds) {
  const int Hs = a.Hs, nh = Hs / 8, k0 = item * 16;
  copy8_batched<W, 8>(
      16 * nh,
      [&](int i) -> const W* {
        const int row = i / nh, c = i - row * nh;
        return (const W*)a.w1 + (size_t)min(k0 + row, a.r - 1) * (a.d + Hs) + a.d + c * 8;
      },
      [&](int i) -> W* {
        const int row = i / nh, c = i - row * nh;
        return lds + (size_t)row * (Hs + 8) + c * 8;
      });
  __syncthreads();
}

// terms of the bottleneck that do not depend on the GRU state: the H half
// W1[:, :d] H_p (precomputed) and b1, for this lane's 4 rows; fetched before
// the state is ready
struct BottleneckPre {
  float4 zh, b1;
};
// The H half summed over its k splits, in split order.  A lane reads only
// rows of its own work item, so the persistent schedule's bottleneck
// workgroups add the splits of their rows once per launch (zh_sum_rows) and
// read the sums (kSummed); the stepwise kernels add them where they read them.
template <class F>
__device__ __forceinline__ float4 zh_splits_sum(const ChainArgs& a, const float* z, F&& ld) {
  const int ns = a.zh_splits;
  float4 v = ld(z);
  float4 t[kMaxZhSplits - 1];
#pragma unroll
  for (int s = 1; s < kMaxZhSplits; ++s) t[s - 1] = ld(z + (size_t)min(s, ns - 1) * a.zh_stride);  // all loads first
#pragma unroll
  for (int s = 1; s < kMaxZhSplits; ++s)
    if (s < ns) {
      v.x += t[s - 1].x;
      v.y += t[s - 1].y;
      v.z += t[s - 1].z;
      v.w += t[s - 1].w;
    }
  return v;
}
// the sums for work item `item` (rows 16 item .. 16 item + 15) at every
// sequence and position, by the whole workgroup, into zh_sum
__device__ __forceinline__ void zh_sum_rows(const ChainArgs& a, int item) {
  const int n = a.B * a.P * 4;  // (sequence, position, group of four rows)
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int bp = i >> 2, k = item * 16 + (i & 3) * 4;
    if (k < a.r) {
      const size_t o = (size_t)bp * a.r + k;
      const float4 v = zh_splits_sum(a, a.zh + o, [](const float* q) { return *reinterpret_cast<const float4*>(q); });
      *reinterpret_cast<float4*>(a.zh_sum + o) = v;
    }
  }
  __syncthreads();
}
// (sequences seq0 .. seq0 + 16 NCB - 1)
template <int NCB, bool kSummed = false>
__device__ __forceinline__ BottleneckPre bottleneck_pre(const ChainArgs& a, int p, int item, int seq0 = 0) {
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  BottleneckPre q;
  q.zh = make_float4(0.f, 0.f, 0.f, 0.f);
  q.b1 = q.zh;
  const int b = seq0 + wv * 16 + row, k = item * 16 + kg * 4;
  if (wv < NCB && b < a.B && k < a.r) {  // r is a multiple of 8: k..k+3 are valid together
    const size_t o = ((size_t)b * a.P + p) * a.r + k;
    if (a.zh_splits == 1)
      q.zh = *reinterpret_cast<const float4*>(&a.zh[o]);
    else if (kSummed)
      q.zh = *reinterpret_cast<const float4*>(&a.zh_sum[o]);
    else
      q.zh = zh_splits_sum(a, a.zh + o, [](const float* z) { return *reinterpret_cast<const float4*>(z); });
    if (a.b1) q.b1 = *reinterpret_cast<const float4*>(&a.b1[k]);
  }
  return q;
}

// The bottleneck's pre-activations are sums over k chunks of 32 in the same
// sixteen chains as the GRU's: chain v takes the chunks c with c % 16 == v in
// increasing order, and the total is ((zh + b1) + F0) + F1 + F2 + F3 (left to
// right) with Fw = ((chain w + chain w+4) + chain w+8) + chain w+12.  With
// NWV = 4 waves, wave w keeps chains w, w+4, w+8, w+12 and folds them itself;
// with 8 (16), wave w keeps chains w and w+8 (chain w) and the fold reads
// every chain from LDS (red: 16 NCB float4 per lane); the sums are the same
// bits.
// kLL: state in and activations out as hand-off words of the persistent launch
// `ep`; with h_s (LDS, B * Hs words) the whole workgroup polls the state
// words once and the waves read their fragments from there.  kOutLL (stepwise
// schedule with phase W inside the phase-O launch): the state from the
// stepwise buffer, the activations out as hand-off words of launch `ep`.
template <class W, int NCB, bool kLdsW, bool kLL = false, int NWV = 4, bool kOutLL = kLL>
__device__ __forceinline__ void bottleneck_item(const ChainArgs& a, int p, int item, float* red, const W* w1_lds,
                                const BottleneckPre& pre_terms, uint32_t ep = 0, uint32_t* h_s = nullptr,
                                int seq0 = 0, int seq_end = kMaxChainGroup) {
  static_assert(NWV == 4 || NWV == 8 || NWV == 16, "four, eight or sixteen waves");
  static_assert(!kLL || kOutLL, "hand-off words in, hand-off words out");
  constexpr int NC = 16 / NWV;  // chains per wave: wv, wv + NWV, ...
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int Hs = a.Hs, B = a.B, r = a.r;
  const int bend = min(B, seq_end);  // columns from seq_end on are left out
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
    const int b = seq0 + cb * 16 + row;
    bok[cb] = b < bend;
    bb[cb] = bok[cb] ? b : 0;
  }
  f32x4 acc[NC][NCB];
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[j][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // chunks per batch, a multiple of NC: chunk c0 + NWV q is in this wave's chain q % NC
  constexpr int U = NWV == 16 ? 2 : (NWV == 8 ? 4 : (NCB == 1 ? 8 : 4));
  const int nch = (Hs + 31) / 32;
  if (kLL && h_s) stage_words_ll(a.status, a.ll_h + (size_t)(p + 1) * B * Hs, B * Hs, ll_tag(ep, p), h_s);
  DH_STAMP(p, 10);
  for (int c0 = wv; c0 < nch; c0 += NWV * U) {  // this wave's chunks wv, wv + NWV, ... in order
    frag_t<W> A[U];
    typename act<W>::type S[U][NCB];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int c = c0 + NWV * q, k = c * 32;
      const bool kok = c < nch && k + kg * 8 < Hs;
      A[q] = load8_or_zero(rw + k, kok);
      if (kLL && h_s) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) S[q][cb] = staged_frag<W>(h_s, Hs, bb[cb], k + kg * 8, kok && bok[cb]);
      } else if constexpr (!kLL) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) S[q][cb] = state_frag<W>(a, p + 1, bb[cb], k + kg * 8, kok && bok[cb]);
      }
    }
    if (kLL && !h_s) {
      const uint64_t* slot = a.ll_h + (size_t)(p + 1) * B * Hs;
      ll_wait(a.status, [&] {
        bool good = true;
#pragma unroll
        for (int q = 0; q < U; ++q) {
          const int c = c0 + NWV * q, k = c * 32;
          const bool kok = c < nch && k + kg * 8 < Hs;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            good = ll_frag<W>(slot, Hs, bb[cb], k + kg * 8, ll_tag(ep, p), kok && bok[cb], S[q][cb]) & good;
        }
        return good;
      });
      DH_STAMP(p, 11);
    }
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[q % NC][cb] = mma(A[q], S[q][cb], acc[q % NC][cb]);
  }
  DH_STAMP(p, 9);
  auto red4 = [&](int e, int cb) -> float4& { return *reinterpret_cast<float4*>(&red[((e * NCB + cb) * 64 + lane) * 4]); };
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    if constexpr (NWV == 4) {  // this wave's fold F_wv
      const f32x4 f = ((acc[0][cb] + acc[1][cb]) + acc[2][cb]) + acc[3][cb];
      red4(wv, cb) = make_float4(f[0], f[1], f[2], f[3]);
    } else {  // chains wv, wv + NWV, ...
#pragma unroll
      for (int j = 0; j < NC; ++j) red4(wv + NWV * j, cb) = make_float4(acc[j][cb][0], acc[j][cb][1], acc[j][cb][2], acc[j][cb][3]);
    }
  }
  __syncthreads();
  if (wv < NCB) {
    const int cb = wv;
    float pre[4] = {pre_terms.zh.x + pre_terms.b1.x, pre_terms.zh.y + pre_terms.b1.y,
                    pre_terms.zh.z + pre_terms.b1.z, pre_terms.zh.w + pre_terms.b1.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float4 v = red4(w, cb);
      if constexpr (NWV != 4) {
#pragma unroll
        for (int j = 1; j < 4; ++j) {
          const float4 u = red4(w + 4 * j, cb);
          v = make_float4(v.x + u.x, v.y + u.y, v.z + u.z, v.w + u.w);
        }
      }
      pre[0] += v.x;
      pre[1] += v.y;
      pre[2] += v.z;
      pre[3] += v.w;
    }
    const int b = seq0 + cb * 16 + row, k = k0 + kg * 4;
    if (b < bend && k < r) {  // r is a multiple of 8, so k..k+3 are all valid
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = pre[i] / (1.f + expf(-pre[i]));
      char* slot = (char*)a.act + (size_t)p * a.act_step;
      if constexpr (kOutLL) {
        ll_put4<W>(a.ll_act + (size_t)p * B * r, r, b, k, s, ll_tag(ep, p));
      } else if constexpr (sizeof(W) == 2) {
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
constexpr int kOEarly = 2;  // tiles of phase O issued before the activations are ready
constexpr int kWShare = 3;  // W2 share of a bottleneck workgroup, in eighths of the others'

// Running argmax of one lane over the logits it has seen, in increasing
// vocabulary order: the value and index of its first maximum (i < 0: none
// yet).  -0 and +0 compare equal; the packed key is formed once at the end.
struct LaneMax {
  float v;
  int32_t i;
};
__device__ __forceinline__ void lane_max(LaneMax& m, float L, int32_t idx, bool valid = true) {
  const bool take = valid & ((L > m.v) | (m.i < 0));  // no short circuit: selects, not branches
  m.v = take ? L : m.v;
  m.i = take ? idx : m.i;
}
__device__ __forceinline__ uint64_t lane_key(const LaneMax& m) { return m.i < 0 ? 0 : amax_key(m.v, (uint32_t)m.i); }

// W2 tiles of workgroup `wg`: the bottleneck workgroups start phase O late,
// so they take a smaller share (kWShare / 8 of the others').
__host__ __device__ inline void o_tile_range(int wg, int G, int nW, int T, int& t_begin, int& t_end) {
  const int64_t wsh = kWShare, units = (int64_t)nW * wsh + (int64_t)(G - nW) * 8;
  auto start_of = [&](int w) -> int64_t {
    const int64_t u = w <= nW ? (int64_t)w * wsh : (int64_t)nW * wsh + (int64_t)(w - nW) * 8;
    return (int64_t)T * u / units;
  };
  t_begin = (int)start_of(wg);
  t_end = (int)start_of(wg + 1);
}

// Resident W2.  Of a workgroup's tiles [t_begin, t_end) the first 4*NTW live
// in registers for all P steps (wave wv owns t_begin + wv + 4i, i < NTW, as
// MFMA right operands) and the rest, at most kLdsTiles, in LDS in fragment
// order (tile j, k chunk c, lane l at 16-byte slot (j*KC + c)*64 + l, so a
// wave's fragment read is 1 KB contiguous).  Slot i of wave wv is tile
// t_begin + wv + 4i throughout.  Phase O then reads no weights from memory.
constexpr int kLdsTilesPerWave = 5;
constexpr int kLdsTiles = 4 * kLdsTilesPerWave;
template <int KC>
constexpr int resident_tiles() {  // 4 AGPRs per lane per k chunk; at most 192 of them, so the rest fits
  return KC >= 8 ? 6 : (KC >= 4 ? 10 : 8);
}
template <class W, int KC>
constexpr bool resident_fits() {
  return sizeof(W) == 2 && KC <= 8;
}
__host__ __device__ inline size_t w2_lds_tile_bytes(int KC) { return (size_t)KC * 64 * 16; }

// Loads from clamped, in-bounds addresses (no select).  Rows past V are never
// stored; k positions past r meet zero activations, so the finite weights
// read there add exactly zero.
// Staged activations in LDS, one row of act_row_words words per sequence.
// bf16 weights: the hi words (bf16 pairs) of sequence b at b*S + q, q < r/2,
// its lo words at b*S + P + 4 + q, where P = 16 KC >= r/2 and S = 2P + 8; the
// 4-word shift puts the 16 (sequence, half) rows of one fragment read in
// distinct banks.  fp32 weights: the values at b*S + q, S = 32 KC + 8.  Words
// from r/2 (fp32: r) up to the k chunks' end hold zeros, so fragment reads
// need no bounds: the pads are cleared once per launch (act_clear_pads).
__host__ __device__ constexpr int act_half_words(int kc, int wsize) { return wsize == 2 ? 16 * kc : 32 * kc; }
__host__ __device__ constexpr int act_row_words(int kc, int wsize) {
  return wsize == 2 ? 2 * act_half_words(kc, 2) + 8 : act_half_words(kc, 4) + 8;
}
__host__ __device__ inline size_t act_stage_bytes(int B, int kc, int wsize) {
  return ((size_t)B * act_row_words(kc, wsize) * 4 + 255) & ~size_t(255);
}
// LDS bytes of B * n staged 32-bit words
__host__ __device__ inline size_t stage_words_bytes(int B, int n) { return ((size_t)B * n * 4 + 255) & ~size_t(255); }
// word q (< r for fp32; bf16: hi words q < r/2, then lo words) of sequence b
template <class W, int KC>
__device__ __forceinline__ int act_stage_index(int q, int b, int r) {
  constexpr int P = act_half_words(KC, sizeof(W)), S = act_row_words(KC, sizeof(W));
  if constexpr (sizeof(W) == 2) return b * S + (q < r / 2 ? q : q - r / 2 + P + 4);
  return b * S + q;
}
template <class W, int KC>
__device__ __forceinline__ void act_clear_pads(uint32_t* act_s, int B, int r) {
  constexpr int P = act_half_words(KC, sizeof(W)), S = act_row_words(KC, sizeof(W));
  const int used = sizeof(W) == 2 ? r / 2 : r, pad = P - used;
  if (pad <= 0) return;
  for (int q = threadIdx.x; q < B * pad; q += blockDim.x) {
    const int b = q / pad, w = used + q % pad;
    act_s[b * S + w] = 0u;
    if constexpr (sizeof(W) == 2) act_s[b * S + P + 4 + w] = 0u;
  }
}

// (t may be -1 for a workgroup that owns no tile; such rows are never used)
template <class W>
__device__ __forceinline__ const W* w2_frag_ptr(const ChainArgs& a, int t, int row, int kg, int c) {
  const int v = min(max(t * 16 + row, 0), a.V - 1);
  return (const W*)a.w2 + (size_t)v * a.r + min(c * 32 + kg * 8, a.r - 8);
}

// The register tier is loaded straight into AGPRs (the MFMA reads its right
// operand from there), so it does not compete with the VGPRs the phases use.
// The loads are not visible to the compiler's wait-count tracking, hence the
// explicit wait for all of them; later compiler-issued waits are only ever
// stricter while these are outstanding, since loads retire in order.
// Eight 16-byte loads straight into AGPRs; the wait for them is part of the
// same asm statement, so no output register is seen by the compiler before
// its data has landed.
__device__ __forceinline__ void agpr_load8(bf16x8* o, const void* const (&p)[8]) {
  asm volatile(
      "global_load_dwordx4 %0, %8, off\n\t"
      "global_load_dwordx4 %1, %9, off\n\t"
      "global_load_dwordx4 %2, %10, off\n\t"
      "global_load_dwordx4 %3, %11, off\n\t"
      "global_load_dwordx4 %4, %12, off\n\t"
      "global_load_dwordx4 %5, %13, off\n\t"
      "global_load_dwordx4 %6, %14, off\n\t"
      "global_load_dwordx4 %7, %15, off\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&a"(o[0]), "=&a"(o[1]), "=&a"(o[2]), "=&a"(o[3]), "=&a"(o[4]), "=&a"(o[5]), "=&a"(o[6]), "=&a"(o[7])
      : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7])
      : "memory");
}
// The same for sixteen loads (two tiles): fewer waits at the start of the launch.
__device__ __forceinline__ void agpr_load16(bf16x8* o, const void* const (&p)[16]) {
  asm volatile(
      "global_load_dwordx4 %0, %16, off\n\t"
      "global_load_dwordx4 %1, %17, off\n\t"
      "global_load_dwordx4 %2, %18, off\n\t"
      "global_load_dwordx4 %3, %19, off\n\t"
      "global_load_dwordx4 %4, %20, off\n\t"
      "global_load_dwordx4 %5, %21, off\n\t"
      "global_load_dwordx4 %6, %22, off\n\t"
      "global_load_dwordx4 %7, %23, off\n\t"
      "global_load_dwordx4 %8, %24, off\n\t"
      "global_load_dwordx4 %9, %25, off\n\t"
      "global_load_dwordx4 %10, %26, off\n\t"
      "global_load_dwordx4 %11, %27, off\n\t"
      "global_load_dwordx4 %12, %28, off\n\t"
      "global_load_dwordx4 %13, %29, off\n\t"
      "global_load_dwordx4 %14, %30, off\n\t"
      "global_load_dwordx4 %15, %31, off\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&a"(o[0]), "=&a"(o[1]), "=&a"(o[2]), "=&a"(o[3]), "=&a"(o[4]), "=&a"(o[5]), "=&a"(o[6]), "=&a"(o[7]),
        "=&a"(o[8]), "=&a"(o[9]), "=&a"(o[10]), "=&a"(o[11]), "=&a"(o[12]), "=&a"(o[13]), "=&a"(o[14]), "=&a"(o[15])
      : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7]),
        "v"(p[8]), "v"(p[9]), "v"(p[10]), "v"(p[11]), "v"(p[12]), "v"(p[13]), "v"(p[14]), "v"(p[15])
      : "memory");
}
__device__ __forceinline__ void agpr_load1(bf16x8& o, const void* p) {
  asm volatile("global_load_dwordx4 %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=&a"(o) : "v"(p) : "memory");
}

template <class W, int KC, int NTW>
__device__ __forceinline__ void load_resident_w2(const ChainArgs& a, int t_begin, int t_end, frag_t<W> (&w2r)[NTW][KC]) {
  static_assert(sizeof(W) == 2, "resident W2 is bf16");
  const int lane = opaque_lane(), wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  constexpr int N = NTW * KC;  // fragments of this wave, in groups of 8 per asm statement
  auto ptr_of = [&](int f) -> const void* {
    const int i = f / KC, c = f % KC;
    return w2_frag_ptr<W>(a, min(t_begin + wv + 4 * i, t_end - 1), row, kg, c);
  };
  frag_t<W>* flat = &w2r[0][0];
#pragma unroll
  for (int f0 = 0; f0 + 16 <= N; f0 += 16) {
    const void* const p[16] = {ptr_of(f0),      ptr_of(f0 + 1),  ptr_of(f0 + 2),  ptr_of(f0 + 3),
                               ptr_of(f0 + 4),  ptr_of(f0 + 5),  ptr_of(f0 + 6),  ptr_of(f0 + 7),
                               ptr_of(f0 + 8),  ptr_of(f0 + 9),  ptr_of(f0 + 10), ptr_of(f0 + 11),
                               ptr_of(f0 + 12), ptr_of(f0 + 13), ptr_of(f0 + 14), ptr_of(f0 + 15)};
    agpr_load16(flat + f0, p);
  }
#pragma unroll
  for (int f0 = N - N % 16; f0 + 8 <= N; f0 += 8) {
    const void* const p[8] = {ptr_of(f0), ptr_of(f0 + 1), ptr_of(f0 + 2), ptr_of(f0 + 3),
                              ptr_of(f0 + 4), ptr_of(f0 + 5), ptr_of(f0 + 6), ptr_of(f0 + 7)};
    agpr_load8(flat + f0, p);
  }
#pragma unroll
  for (int f = N - N % 8; f < N; ++f) agpr_load1(flat[f], ptr_of(f));
}

// the LDS tier: tiles t_begin + 4*NTW + j, j < n_lds
template <class W, int KC>
__device__ __forceinline__ void stage_w2_lds(const ChainArgs& a, int t_first, int n_lds, unsigned char* lds) {
  static_assert(sizeof(W) == 2, "resident W2 is bf16");
  copy8_batched<W, 13>(
      n_lds * KC * 64,
      [&](int q) {
        const int l = q & 63, c = (q >> 6) % KC, j = q / (KC * 64);
        return w2_frag_ptr<W>(a, t_first + j, l & 15, l >> 4, c);
      },
      [&](int q) { return reinterpret_cast<W*>(lds + (size_t)q * 16); });
  __syncthreads();
}

// ---- phase O in paired-row form --------------------------------------------------
// The MFMA's left operand holds the activations: row 2j of row group g is the
// bf16 hi half of sequence 8g + j, row 2j + 1 its lo half (fp32 weights: the
// value, and zeros).  The right operand is a 16-row W2 tile, so lane l holds,
// for vocabulary entry t*16 + l % 16, result rows 4kg .. 4kg + 3 (kg = l / 16):
// the hi and lo sums of sequences 8g + 2kg and 8g + 2kg + 1.  Eight sequences
// share one MFMA per k chunk, and a lane's epilogue handles one entry.
// L = (Lb + b2) + (hi + lo), hi and lo each the even k chunks' sum plus the
// odd ones'; every phase-O variant computes exactly this.
constexpr int kSeqPerRowGroup = 8;

// left operand, elements k..k+7 (k < 32 KC), for row `row` of row group g.
// Rows of sequences past B read sequence B - 1: their results are never used.
template <class W, int KC>
__device__ __forceinline__ frag_t<W> act_row_frag(const uint32_t* act_s, int B, int g, int row, int k) {
  constexpr int P = act_half_words(KC, sizeof(W)), S = act_row_words(KC, sizeof(W));
  const int b = min(g * kSeqPerRowGroup + (row >> 1), B - 1), part = row & 1;
  const uint32_t* src = act_s + b * S;
  if constexpr (sizeof(W) == 2) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(src + (part ? P + 4 : 0) + k / 2));
  } else {
    f32x8 f;
    f.lo = *reinterpret_cast<const float4*>(src + k);
    f.hi = *reinterpret_cast<const float4*>(src + k + 4);
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    if (part) f.lo = z, f.hi = z;  // the odd rows stay zero for fp32 weights
    return f;
  }
}

// Lb of vocabulary entry v for this lane's sequences (8g + 2kg + j), and b2[v]
// Loads from clamped addresses with no per-lane condition (a lane-dependent
// select here would turn into a masked region that waits for the load, and
// with it for every load issued earlier).  Entries past V are skipped by
// rows_epilogue, rows of sequences past B are never published.  kSkipEmpty:
// rows (g, j) with no sequence in any lane are skipped by a uniform branch;
// inside a software-pipelined loop every load is issued instead, so that the
// number of loads after any given one is fixed and the waits stay exact.
template <int RG, bool kSkipEmpty>
__device__ __forceinline__ void load_base_rows(const ChainArgs& a, int p, int v, int kg, float (&lb)[RG][2],
                                               float& b2) {
  const int vc = min(v, a.V - 1);
  // always loaded (a uniform select of the address); the value is only used
  // when b2 exists (rows_epilogue), so no select here waits for the load
  b2 = (a.b2 ? a.b2 : a.Lb)[vc];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int b = g * kSeqPerRowGroup + 2 * kg + j;
      const float* src = a.Lb + ((size_t)min(b, a.B - 1) * a.P + p) * a.V + vc;
      if constexpr (kSkipEmpty)
        lb[g][j] = g * kSeqPerRowGroup + j < a.B ? *src : 0.f;
      else
        lb[g][j] = *src;
    }
}

// ---- sampling at temperature T (Gumbel-max) ------------------------------------------
// A draw from softmax(L / T) is argmax_v (L_v + T g_v) with g_v standard
// Gumbel noise.  The noise of (sequence b of the whole batch, position p,
// entry v) is -log(-log u), u = (2 (x >> 9) + 1) / 2^24 (exact in fp32),
// x = word (b & 1) of Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011)
// at counter (v, p, b >> 1, 0) under key (seed lo, seed hi): one generator
// call serves the pair of sequences a lane holds in a row group.
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1, uint32_t& x0, uint32_t& x1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  x0 = c0;
  x1 = c1;
}
__device__ __forceinline__ float gumbel_of(uint32_t x) {
  const float u = (float)(2u * (x >> 9) + 1u) * 0x1p-24f;  // exact
  return -logf(-logf(u));
}

// this lane's logits of a tile into its running argmaxes (and out, with
// kWrite); kSample: the argmax is taken over L + T g (the logits written are L)
// (entries past V take part in no argmax and are not written; a select, not a
// branch, so no load is waited for inside a masked region)
template <bool kWrite, int RG, bool kSample = false>
__device__ __forceinline__ void rows_epilogue(const ChainArgs& a, int p, int v, int kg, const float (&lb)[RG][2],
                                              float b2, const f32x4 (&acc)[RG][2], LaneMax (&lm)[RG][2]) {
  const bool valid = v < a.V;
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    uint32_t x[2] = {0u, 0u};
    if constexpr (kSample) {  // the lane's sequences a.seq_base + 8g + 2kg + {0, 1}: one generator call
      const uint32_t pair = (uint32_t)(a.seq_base + g * kSeqPerRowGroup + 2 * kg) >> 1;
      philox4x32_10((uint32_t)v, (uint32_t)p, pair, 0u, a.seed_lo, a.seed_hi, x[0], x[1]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float hi = acc[g][0][2 * j] + acc[g][1][2 * j];
      const float lo = acc[g][0][2 * j + 1] + acc[g][1][2 * j + 1];
      const float base = a.b2 ? lb[g][j] + b2 : lb[g][j];
      const float L = base + (hi + lo);
      if constexpr (kSample)
        lane_max(lm[g][j], L + a.temperature * gumbel_of(x[j]), v, valid);
      else
        lane_max(lm[g][j], L, v, valid);
      if constexpr (kWrite) {
        const int b = g * kSeqPerRowGroup + 2 * kg + j;
        if (valid && b < a.B) a.out_logits[((size_t)b * a.P + p) * a.V + v] = L;
      }
    }
  }
}

// Fold the lanes' running argmaxes into one key per sequence for this
// workgroup, then into the device-wide key of step p (atomic max), or, kLL,
// publish it as this workgroup's (value, index) pair of hand-off words.
template <int RG, bool kLL, int NWV = 4>
__device__ __forceinline__ void publish_rows(const ChainArgs& a, int p, LaneMax (&lm)[RG][2], uint64_t* sbest,
                                             uint32_t ep) {
  const int lane = opaque_lane(), wv = threadIdx.x >> 6, kg = lane >> 4;
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint64_t k = lane_key(lm[g][j]);
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) k = umax64(k, shfl_xor_u64(k, m));  // the 16 lanes of this kg
      if ((lane & 15) == 0) sbest[wv * kMaxChainGroup + g * kSeqPerRowGroup + 2 * kg + j] = k;
    }
  __syncthreads();
  if (threadIdx.x < RG * kSeqPerRowGroup) {
    const int b = threadIdx.x;
    uint64_t m = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) m = umax64(m, sbest[w * kMaxChainGroup + b]);
    if constexpr (kLL) {
      if (b < a.B) {
        uint64_t* w = a.ll_part + (((size_t)p * kMaxChainGrid + blockIdx.x) * a.B + b) * 2;
        ll_put(w, (uint32_t)(m >> 32), ll_tag(ep, p));
        ll_put(w + 1, (uint32_t)m, ll_tag(ep, p));
      }
    } else {
      if (b < a.B && m != 0) atomicMax((unsigned long long*)&a.keys[(size_t)p * a.B + b], (unsigned long long)m);
    }
  }
  __syncthreads();
}

// The bottleneck activations of step p, staged in LDS (act_stage_index).
template <class W, int KC>
__device__ __forceinline__ void stage_act_ll(const ChainArgs& a, int p, uint32_t ep, uint32_t* act_s) {
  const int r = a.r;
  stage_words_ll(a.status, a.ll_act + (size_t)p * a.B * r, a.B * r, ll_tag(ep, p), act_s,
                 [r](int q) { return act_stage_index<W, KC>(q % r, q / r, r); });
}
// the same staging from the stepwise schedule's activation buffer (bf16: hi
// [B][r] then lo [B][r]; fp32: [B][r]), four words per load and every
// thread's loads in flight before its stores (a loop of single
// load-then-store pairs waits one memory round trip per word); indices past
// the end repeat the last piece, as in copy8_batched
template <class W, int KC>
__device__ __forceinline__ void stage_act_global(const ChainArgs& a, int p, uint32_t* act_s) {
  constexpr int NB = 4;  // (the asm below names four)
  const int B = a.B, r = a.r, n4 = B * r / 4;  // r is a multiple of 8
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* slot = reinterpret_cast<const u32x4*>((const char*)a.act + (size_t)p * a.act_step);
  auto dst = [&](int q) {
    const int wq = 4 * q;
    if constexpr (sizeof(W) == 2) {
      const int half = B * (r / 2), lo = wq >= half, rem = wq - (lo ? half : 0);
      const int b = rem / (r / 2), w = rem - b * (r / 2);
      return act_s + act_stage_index<W, KC>(lo ? w + r / 2 : w, b, r);
    } else {
      const int b = wq / r;
      return act_s + act_stage_index<W, KC>(wq - b * r, b, r);
    }
  };
  for (int q0 = 0; q0 < n4; q0 += NB * (int)blockDim.x) {
    u32x4 v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) v[u] = slot[min(q0 + u * (int)blockDim.x + (int)threadIdx.x, n4 - 1)];
    // all four loads issued before the first store (left alone, the scheduler
    // pairs each load with its store, one round trip each)
    asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
#pragma unroll
    for (int u = 0; u < NB; ++u)
      *reinterpret_cast<u32x4*>(dst(min(q0 + u * (int)blockDim.x + (int)threadIdx.x, n4 - 1))) = v[u];
  }
  __syncthreads();
}

// phase O with resident W2 (persistent schedule): the base logits of every
// owned tile are fetched before the activations exist
template <class W, int RG, int KC, int NTW, bool kWrite, bool kSample>
__device__ __forceinline__ void logits_resident_(const ChainArgs& a, int p, int t_begin, int t_end,
                                                 const frag_t<W> (&w2r)[NTW][KC], const unsigned char* w2_lds,
                                                 uint32_t* act_s, uint64_t* sbest, uint32_t ep) {
  constexpr int NT = NTW + kLdsTilesPerWave;  // slots below NTW: registers; then LDS
  const int lane = opaque_lane(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15, kg = lane >> 4;
  auto tile_of = [&](int i) { return t_begin + wv + 4 * i; };
  float lb[NT][RG][2], b2[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) load_base_rows<RG, true>(a, p, tile_of(i) * 16 + row, kg, lb[i], b2[i]);
  stage_act_ll<W, KC>(a, p, ep, act_s);  // the activations of this step
  DH_STAMP(p, 4);
  frag_t<W> af[RG][KC];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int c = 0; c < KC; ++c) af[g][c] = act_row_frag<W, KC>(act_s, a.B, g, row, c * 32 + kg * 8);
  LaneMax lm[RG][2];
#pragma unroll
  for (int g = 0; g < RG; ++g) lm[g][0] = lm[g][1] = LaneMax{0.f, -1};
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    if (tile_of(i) >= t_end) break;
    f32x4 acc[RG][2];
#pragma unroll
    for (int g = 0; g < RG; ++g) acc[g][0] = acc[g][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < NTW) {
#pragma unroll
      for (int c = 0; c < KC; ++c)
#pragma unroll
        for (int g = 0; g < RG; ++g) acc[g][c & 1] = mma(af[g][c], w2r[i < NTW ? i : 0][c], acc[g][c & 1]);
    } else {
      const unsigned char* src = w2_lds + ((size_t)(4 * (i - NTW) + wv) * KC * 64 + lane) * 16;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const frag_t<W> w = *reinterpret_cast<const frag_t<W>*>(src + (size_t)c * 64 * 16);
#pragma unroll
        for (int g = 0; g < RG; ++g) acc[g][c & 1] = mma(af[g][c], w, acc[g][c & 1]);
      }
    }
    rows_epilogue<kWrite, RG, kSample>(a, p, tile_of(i) * 16 + row, kg, lb[i], b2[i], acc, lm);
  }
  DH_STAMP(p, 6);
  publish_rows<RG, true>(a, p, lm, sbest, ep);
  DH_STAMP(p, 7);
}

template <class W, int RG, int KC, int NTW, bool kSample>
__device__ __forceinline__ void logits_resident(const ChainArgs& a, int p, int t_begin, int t_end,
                                                const frag_t<W> (&w2r)[NTW][KC], const unsigned char* w2_lds,
                                                uint32_t* act_s, uint64_t* sbest, uint32_t ep) {
  if (a.out_logits)
    logits_resident_<W, RG, KC, NTW, true, kSample>(a, p, t_begin, t_end, w2r, w2_lds, act_s, sbest, ep);
  else
    logits_resident_<W, RG, KC, NTW, false, kSample>(a, p, t_begin, t_end, w2r, w2_lds, act_s, sbest, ep);
}

template <class W, int RG, int KC>
struct TileBuf {
  frag_t<W> w[KC];  // 16 W2 rows x all of k, MFMA right operand
  float lb[RG][2];  // base logits of this lane's entry for its sequences
  float b2;
};

// phase O with W2 streamed from memory: each wave walks its tiles t_begin +
// wv, + 4, ... with three named tile buffers, two tiles ahead of the one it
// multiplies.  Every pass issues the same loads (past the wave's last tile
// they repeat a valid tile, never used), so the number of loads issued after
// any given one is fixed and the compiler's wait counts cover exactly the
// tile being consumed; a buffer array indexed in a loop would instead be
// rotated through register copies, each of which waits for its load.  The
// first kOEarly tiles are issued before the activations exist (before
// `ready` in the stepwise schedule).
template <class W, int RG, int KC, bool kWrite, bool kLL, class Ready, bool kSample = false>
__device__ __forceinline__ bool logits_range_(const ChainArgs& a, int p, int t_begin, int t_end, uint64_t* sbest,
                                              Ready ready, uint32_t ep, uint32_t* act_s) {
  static_assert(kOEarly >= 0 && kOEarly <= 2, "two tiles ahead");
  const int lane = opaque_lane(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15, kg = lane >> 4;
  const int t0 = t_begin + wv, n = t_end > t0 ? (t_end - t0 + 3) / 4 : 0;  // tiles of this wave
  const int t_last = t_end > t_begin ? t_end - 1 : max(t_begin, 0);
  auto issue = [&](int i, TileBuf<W, RG, KC>& tb) {
    const int t = min(t0 + 4 * i, t_last);
#pragma unroll
    for (int c = 0; c < KC; ++c) tb.w[c] = load8(w2_frag_ptr<W>(a, t, row, kg, c));
    load_base_rows<RG, false>(a, p, t * 16 + row, kg, tb.lb, tb.b2);
  };
  TileBuf<W, RG, KC> s0, s1, s2;
  if (kOEarly >= 1) issue(0, s0);
  if (kOEarly >= 2) issue(1, s1);
  if constexpr (!kLL) {
    if (!ready()) return false;
  }
  if (kOEarly < 1) issue(0, s0);
  if (kOEarly < 2) issue(1, s1);
  if constexpr (kLL)
    stage_act_ll<W, KC>(a, p, ep, act_s);
  else
    stage_act_global<W, KC>(a, p, act_s);
  // left operands kept in registers when they fit in 64, else read per tile from LDS
  constexpr bool kAfRegs = RG * KC * (int)(sizeof(frag_t<W>) / 4) <= 64;
  frag_t<W> af[kAfRegs ? RG : 1][kAfRegs ? KC : 1];
  if constexpr (kAfRegs) {
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int c = 0; c < KC; ++c) af[g][c] = act_row_frag<W, KC>(act_s, a.B, g, row, c * 32 + kg * 8);
  }
  LaneMax lm[RG][2];
#pragma unroll
  for (int g = 0; g < RG; ++g) lm[g][0] = lm[g][1] = LaneMax{0.f, -1};
  auto consume = [&](int i, const TileBuf<W, RG, KC>& tb) {
    f32x4 acc[RG][2];  // even and odd k chunks: two independent MFMA chains per row group
#pragma unroll
    for (int g = 0; g < RG; ++g) acc[g][0] = acc[g][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        if constexpr (kAfRegs)
          acc[g][c & 1] = mma(af[g][c], tb.w[c], acc[g][c & 1]);
        else
          acc[g][c & 1] = mma(act_row_frag<W, KC>(act_s, a.B, g, row, c * 32 + kg * 8), tb.w[c], acc[g][c & 1]);
      }
    rows_epilogue<kWrite, RG, kSample>(a, p, (t0 + 4 * i) * 16 + row, kg, tb.lb, tb.b2, acc, lm);
  };
  int i = 0;
  for (; i + 3 <= n; i += 3) {
    issue(i + 2, s2);
    consume(i, s0);
    issue(i + 3, s0);
    consume(i + 1, s1);
    issue(i + 4, s1);
    consume(i + 2, s2);
  }
  if (i < n) consume(i, s0);
  if (i + 1 < n) consume(i + 1, s1);
  publish_rows<RG, kLL>(a, p, lm, sbest, ep);
  return true;
}

// phase O of the stepwise schedule with many waves: each of NWV waves takes
// the workgroup's tiles t_begin + wv, + NWV, ... with the next tile's loads in
// flight while it multiplies one (two named buffers, loads always issued from
// clamped addresses so the waits stay exact), and re-reads the staged
// activations from LDS per tile, so it needs few registers and the other
// waves hide what latency is left.  With two row groups (9 to 16 sequences)
// the registers hold a third buffer and each wave runs two tiles ahead
// (495 -> 476 us per block at 16 sequences); with one row group the sixteen
// waves of a workgroup, and with four the tile's row groups, leave no room
// for it (at four the third buffer spilled and cost 603 -> 616 us).
// (kLL: the activations come as hand-off words of launch ep, else from the
// stepwise activation buffer)
template <class W, int RG, int KC, int NWV, bool kWrite, bool kSample = false, bool kLL = false>
__device__ __forceinline__ void logits_wide_(const ChainArgs& a, int p, int t_begin, int t_end, uint64_t* sbest,
                                             uint32_t* act_s, uint32_t ep = 0) {
  const int lane = opaque_lane(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15, kg = lane >> 4;
  const int t0 = t_begin + wv, n = t_end > t0 ? (t_end - t0 + NWV - 1) / NWV : 0;
  const int t_last = t_end > t_begin ? t_end - 1 : max(t_begin, 0);
  auto issue = [&](int i, TileBuf<W, RG, KC>& tb) {
    const int t = min(t0 + NWV * i, t_last);
#pragma unroll
    for (int c = 0; c < KC; ++c) tb.w[c] = load8(w2_frag_ptr<W>(a, t, row, kg, c));
    load_base_rows<RG, false>(a, p, t * 16 + row, kg, tb.lb, tb.b2);
  };
  constexpr bool kAhead2 = RG == 2;
  TileBuf<W, RG, KC> s0, s1, s2;
  issue(0, s0);
  if constexpr (kAhead2) issue(1, s1);
  if constexpr (kLL)
    stage_act_ll<W, KC>(a, p, ep, act_s);
  else
    stage_act_global<W, KC>(a, p, act_s);
  LaneMax lm[RG][2];
#pragma unroll
  for (int g = 0; g < RG; ++g) lm[g][0] = lm[g][1] = LaneMax{0.f, -1};
  auto consume = [&](int i, const TileBuf<W, RG, KC>& tb) {
    const uint32_t* as = act_s + opaque_zero();
    f32x4 acc[RG][2];
#pragma unroll
    for (int g = 0; g < RG; ++g) acc[g][0] = acc[g][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int g = 0; g < RG; ++g)
        acc[g][c & 1] = mma(act_row_frag<W, KC>(as, a.B, g, row, c * 32 + kg * 8), tb.w[c], acc[g][c & 1]);
    rows_epilogue<kWrite, RG, kSample>(a, p, (t0 + NWV * i) * 16 + row, kg, tb.lb, tb.b2, acc, lm);
  };
  int i = 0;
  if constexpr (kAhead2) {
    for (; i + 3 <= n; i += 3) {
      issue(i + 2, s2);
      consume(i, s0);
      issue(i + 3, s0);
      consume(i + 1, s1);
      issue(i + 4, s1);
      consume(i + 2, s2);
    }
    if (i < n) consume(i, s0);
    if (i + 1 < n) consume(i + 1, s1);
  } else {
    for (; i + 2 <= n; i += 2) {
      issue(i + 1, s1);
      consume(i, s0);
      issue(i + 2, s0);
      consume(i + 1, s1);
    }
    if (i < n) consume(i, s0);
  }
  publish_rows<RG, false, NWV>(a, p, lm, sbest, 0u);
}

template <class W, int RG, int KC, bool kLL, class Ready>
__device__ __forceinline__ bool logits_range(const ChainArgs& a, int p, int t_begin, int t_end, uint64_t* sbest,
                                             Ready ready, uint32_t ep, uint32_t* act_s) {
  if (a.out_logits) return logits_range_<W, RG, KC, true, kLL>(a, p, t_begin, t_end, sbest, ready, ep, act_s);
  return logits_range_<W, RG, KC, false, kLL>(a, p, t_begin, t_end, sbest, ready, ep, act_s);
}

// ---- the tokens of a step from the workgroups' argmax pairs ---------------------
// Every workgroup publishes, per sequence, its best (value, index) as a pair
// of hand-off words.  One workgroup per sequence reduces it over the grid and
// publishes the result as one more pair, which the readers poll: two
// hand-offs, but each reader polls B pairs instead of grid x B (letting every
// reader reduce all pairs itself measured slower: the polling traffic of 256
// readers delays everyone).  Tokens are raw argmax indices, as the packed key
// gives them.
__device__ __forceinline__ uint64_t pair_key(uint64_t hi, uint64_t lo) {
  return ((uint64_t)ll_data(hi) << 32) | ll_data(lo);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = umax64(v, shfl_xor_u64(v, m));
  return v;
}

// The last B workgroups of the grid (no bottleneck work, so they reach this
// first) reduce one sequence each of step p and publish it.
__device__ __forceinline__ void ll_tokens_reduce(const ChainArgs& a, int p, uint32_t ep, uint64_t* sred) {
  const int B = a.B, b = (int)gridDim.x - 1 - (int)blockIdx.x;
  if (b < 0 || b >= B) return;
  const int tid = threadIdx.x, wv = tid >> 6;
  const uint32_t tag = ll_tag(ep, p);
  const uint64_t* part = a.ll_part + (size_t)p * kMaxChainGrid * B * 2;
  uint64_t key = 0;
  ll_wait(a.status, [&] {
    bool good = true;
    key = 0;
    for (int w = tid; w < (int)gridDim.x; w += blockDim.x) {
      const uint64_t hi = ld_agent64(part + ((size_t)w * B + b) * 2), lo = ld_agent64(part + ((size_t)w * B + b) * 2 + 1);
      good = good & (int)ll_ok(hi, tag) & (int)ll_ok(lo, tag);
      key = umax64(key, pair_key(hi, lo));
    }
    return good;
  });
  DH_STAMP(p, 14);
  key = wave_max_u64(key);
  if ((tid & 63) == 0) sred[wv] = key;
  __syncthreads();
  if (tid == 0) {
    uint64_t m = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m = umax64(m, sred[w]);
    ll_put(a.ll_tok + ((size_t)p * B + b) * 2, (uint32_t)(m >> 32), tag);
    ll_put(a.ll_tok + ((size_t)p * B + b) * 2 + 1, (uint32_t)m, tag);
  }
  __syncthreads();
}

// tok[b] (LDS) = the token drafted at step p for every sequence b
__device__ __forceinline__ void ll_tokens_read(const ChainArgs& a, int p, uint32_t ep, int32_t* tok) {
  const int B = a.B, lane = threadIdx.x & 63;
  const uint32_t tag = ll_tag(ep, p);
  if (threadIdx.x < 64) {  // B <= kMaxChainGroup <= 64
    uint64_t m = 0;
    ll_wait(a.status, [&] {
      if (lane >= B) return true;
      const uint64_t hi = ld_agent64(a.ll_tok + ((size_t)p * B + lane) * 2);
      const uint64_t lo = ld_agent64(a.ll_tok + ((size_t)p * B + lane) * 2 + 1);
      m = pair_key(hi, lo);
      return ll_ok(hi, tag) && ll_ok(lo, tag);
    });
    if (lane < B) tok[lane] = amax_index(m);
  }
  __syncthreads();
}

// ---- kernels ------------------------------------------------------------------------
// Before the steps: the H half of the bottleneck for every position,
// zh[b][p][k] = sum_i H[b][p][i] W1[k][i], and the zeroed keys and initial
// state.  One 16x16 tile per workgroup and k split (blockIdx.z) over the
// waves; split s writes its partial sum to zh + s * zh_stride (with few
// tiles the splits spread one tile's k range over many CUs, whose fetch
// rate bounds this kernel).
template <class W>
__global__ __launch_bounds__(256) void chain_prologue(ChainArgs a, const void* H, int reset_status) {
  __shared__ __attribute__((aligned(16))) float red[4 * 64 * 4];
  const int M = a.B * a.P;
  const int nblk = gridDim.x * gridDim.y * gridDim.z, blk = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
  const int tid = blk * blockDim.x + threadIdx.x, stride = nblk * blockDim.x;
  if (blk == 0) {
    // The launch's bookkeeping, every read in flight at once (a chain of
    // dependent reads costs a memory round trip each).  First launch on this
    // workspace, or on a different layout of it, or the launch counter about
    // to overflow the tags: clear the hand-off words, so that no leftover bits
    // can carry a current tag; between clears the launch counter alone keeps
    // earlier launches' words from passing.  Out-of-range first tokens set
    // status 1 unless a status is already set.
    __shared__ int fresh, status_in;
    __shared__ uint32_t epoch_in;
    if (threadIdx.x == 0) {
      const uint64_t mk = *a.marker, sg = *a.sig;
      const uint32_t ep = *a.epoch;
      const int32_t st = *a.status;
      fresh = mk != kLLMarker || sg != a.sig_value || ep + 1 >= kEpochLimit;
      epoch_in = ep;
      status_in = reset_status ? 0 : st;
    }
    const int b = threadIdx.x;  // B <= kMaxChainGroup <= blockDim
    const int bad = __syncthreads_or(b < a.B && (a.t0[b] < 0 || a.t0[b] >= a.V));
    if (fresh) {
      uint4* w = reinterpret_cast<uint4*>(a.ll_h);
      for (size_t i = threadIdx.x; i < a.ll_words / 2; i += blockDim.x) w[i] = make_uint4(0, 0, 0, 0);
      if (threadIdx.x == 0) {
        *a.marker = kLLMarker;
        *a.sig = a.sig_value;
      }
    }
    if (threadIdx.x == 0) {
      *a.epoch = (fresh ? 0u : epoch_in) + 1u;  // tags of this launch's hand-off words
      *a.status = status_in == 0 && bad ? 1 : status_in;
    }
  }
  if (a.zh_splits == 1) {
    splitk_tile<W>((const W*)H, a.d, (const W*)a.w1, a.d + a.Hs, (float*)a.zh, a.r, M, a.r, a.d, blockIdx.x, blockIdx.y,
                   red);
  } else {
    const int nck = (a.d + 31) / 32, per = (nck + a.zh_splits - 1) / a.zh_splits, s = blockIdx.z;
    const int cb = min(s * per, nck), ce = min(cb + per, nck);
    splitk_tile_n<W, 4, 4>((const W*)H, a.d, (const W*)a.w1, a.d + a.Hs, (float*)a.zh + (size_t)s * a.zh_stride, a.r,
                           M, a.r, a.d, blockIdx.x, blockIdx.y, red, cb, ce);
  }
  for (int i = tid; i < a.P * a.B; i += stride) a.keys[i] = 0;
  for (int i = tid; i < a.B * a.Hs; i += stride) a.h[i] = 0.f;  // state slot 0
}

__global__ void chain_finalize(ChainArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < a.B * a.P) {
    const int b = i / a.P, p = i % a.P;
    a.out_tokens[i] = amax_index(a.keys[(size_t)p * a.B + b]);
  }
}

// Three-launch schedule, phase G: work item = 4 units, all sequences.
// (Splitting the sequences over workgroups, 16 per workgroup, measured
// slower at 32 sequences: 16.4 against 14.9 us per step.)
template <class W, int NCB, bool kTab>
__global__ __launch_bounds__(256) void chain_gru_k(ChainArgs a, int p) {
  __shared__ __attribute__((aligned(16))) float red[4 * NCB * 64 * 4];
  for (int it = blockIdx.x; it < a.Hs / 4; it += gridDim.x) {
    f32x4 acc_h[4][NCB];
    gru_hidden_part<W, NCB, false>(a, p, it, nullptr, acc_h);
    gru_finish<W, NCB, false, false, kTab>(a, p, it, red, nullptr, acc_h);
  }
}

// Three-launch schedule, phase G with sixteen waves: one work item per
// workgroup, wave v computes GRU chain v (chunks v, v + 16, ... of the hidden
// half, then of the input half), the first batches of both halves loaded
// together; the same sums as the four-wave form.  (Staging the work item's
// weight rows in LDS with whole-row loads first measured slower at 32
// sequences, 17.3 against 14.1 us: the time goes to the sequences' state and
// embedding fragments, which every workgroup reads.)
constexpr int kGru16UH = 2;  // hidden-half chunks per wave per batch (Hs <= 1024 in one batch)
// kStage (with the per-token table, when the state fits): the workgroup first
// copies the split state of every sequence (hi and lo rows of Hs bf16 each)
// into LDS with whole-row loads, rows padded by 8 elements, and the waves read
// their fragments from there: every workgroup reads the same state, and
// fragment-shaped reads of it from L2 are several times slower.  The chains'
// partial sums then reuse the same LDS.
__host__ __device__ inline size_t gru16_stage_bytes(int B, int Hs, int NCB) {
  const size_t st = (size_t)2 * B * (Hs + 8) * 2, red = (size_t)kGruChains * NCB * 64 * 16;
  return st > red ? st : red;
}
template <class W, int NCB, bool kTab, bool kStage = false>
__global__ __launch_bounds__(1024) void chain_gru16_k(ChainArgs a, int p) {
  static_assert(sizeof(W) == 2, "bf16 weights (fp32 fragments need twice the registers)");
  static_assert(!kStage || kTab, "the staged state with the per-token table only");
  // input-half chunks per wave per batch: d <= 2560 in one batch for 16 sequences, two batches for 32
  constexpr int kGru16UX = NCB == 1 ? 5 : 4;
  __shared__ __attribute__((aligned(16))) float red_st[kStage ? 4 : kGruChains * NCB * 64 * 4];
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];  // kStage: the state, then the sums
  float* red = kStage ? reinterpret_cast<float*>(dyn_lds) : red_st;
  const W* hs = reinterpret_cast<const W*>(dyn_lds);
  const int item = blockIdx.x;
  const int lane = opaque_lane(), v = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int d = a.d, Hs = a.Hs, B = a.B;
  const W *rx, *rh;
  bool has_x, has_h;
  gru_rows<W, false>(a, item, nullptr, rx, rh, has_x, has_h);
  int bb[NCB];
  bool bok[NCB];
  const W* xe[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int b = cb * 16 + row;
    bok[cb] = b < B;
    bb[cb] = bok[cb] ? b : 0;
    xe[cb] = (const W*)a.embed + (size_t)(bok[cb] ? prev_token(a, p, b) : 0) * d + kg * 8;
  }
  const int nch = (Hs + 31) / 32, ncx = (d + 31) / 32;
  const bool hid = p > 0;  // h(0) = 0: no hidden half at the first step
  const int SR = Hs + 8;   // staged row stride
  if constexpr (kStage) {
    if (hid) {
      const int per = Hs / 8;
      const uint16_t* src = a.hb + (size_t)p * a.hb_step;  // hi rows [B][Hs], then lo rows
      copy8_batched<W, 8>(2 * B * per, [&](int q) { return (const W*)src + (size_t)q * 8; },
                          [&](int q) {
                            const int r = q / per;
                            return (W*)dyn_lds + (size_t)r * SR + (size_t)(q - r * per) * 8;
                          });
      __syncthreads();
    }
  }
  f32x4 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  frag_t<W> AH[kGru16UH], AX[kGru16UX];
  typename act<W>::type SH[kGru16UH][NCB];
  frag_t<W> XX[kGru16UX][NCB];
  auto load_h = [&](int c0) {
#pragma unroll
    for (int q = 0; q < kGru16UH; ++q) {
      const int c = c0 + 16 * q, k = c * 32;
      const bool kok = hid && c < nch && k + kg * 8 < Hs;
      AH[q] = load8_or_zero(rh + k, kok && has_h);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        if constexpr (kStage) {
          SH[q][cb].hi = load8_or_zero(hs + (size_t)bb[cb] * SR + k + kg * 8, kok && bok[cb]);
          SH[q][cb].lo = load8_or_zero(hs + (size_t)(B + bb[cb]) * SR + k + kg * 8, kok && bok[cb]);
        } else {
          SH[q][cb] = state_frag<W>(a, p, bb[cb], k + kg * 8, kok && bok[cb]);
        }
      }
    }
  };
  auto load_x = [&](int c0) {
#pragma unroll
    for (int q = 0; q < kGru16UX; ++q) {
      const int c = c0 + 16 * q, k = c * 32;
      const bool kok = c < ncx && k + kg * 8 < d;
      AX[q] = load8_or_zero(rx + k, kok && has_x);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) XX[q][cb] = load8_or_zero(xe[cb] + k, kok && bok[cb]);
    }
  };
  // chunks past the end load zeros and add exact zeros, as in the four-wave form
  auto mma_h = [&]() {
#pragma unroll
    for (int q = 0; q < kGru16UH; ++q)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma(AH[q], SH[q][cb], acc[cb]);
  };
  auto mma_x = [&]() {
#pragma unroll
    for (int q = 0; q < kGru16UX; ++q)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma(AX[q], XX[q][cb], acc[cb]);
  };
  // kTab: the input half from the per-token table
  const float4 xin = kTab ? gru_table_in<NCB>(a, p, item, nullptr) : float4{0.f, 0.f, 0.f, 0.f};
  if (hid) load_h(v);
  if (!kTab) load_x(v);
  if (hid) {
    mma_h();
    for (int c0 = v + 16 * kGru16UH; c0 < nch; c0 += 16 * kGru16UH) {
      load_h(c0);
      mma_h();
    }
  }
  if (!kTab) {
    mma_x();
    for (int c0 = v + 16 * kGru16UX; c0 < ncx; c0 += 16 * kGru16UX) {
      load_x(c0);
      mma_x();
    }
  }
  if constexpr (kStage) __syncthreads();  // the sums take the staged state's place
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
    *reinterpret_cast<float4*>(&red[((v * NCB + cb) * 64 + lane) * 4]) = make_float4(acc[cb][0], acc[cb][1], acc[cb][2], acc[cb][3]);
  float h_dummy = 0.f;
  gru_apply<W, NCB, false, 16, kTab>(a, p, item, red, h_dummy, 0u, 0, xin);
}

template <class W, int NCB>
// (blockIdx.y: the block of 16 NCB sequences)
__global__ __launch_bounds__(256) void chain_bottleneck_k(ChainArgs a, int p, int seqs) {
  __shared__ __attribute__((aligned(16))) float red[4 * NCB * 64 * 4];
  const int seq0 = blockIdx.y * seqs;
  for (int it = blockIdx.x; it < (a.r + 15) / 16; it += gridDim.x)
    bottleneck_item<W, NCB, false>(a, p, it, red, nullptr, bottleneck_pre<NCB>(a, p, it, seq0), 0u, nullptr, seq0,
                                   seq0 + seqs);
}

template <class W, int RG, int KC, bool kSample>
__global__ __launch_bounds__(256) void chain_logits_k(ChainArgs a, int p) {
  __shared__ uint64_t sbest[4 * kMaxChainGroup];
  __shared__ __attribute__((aligned(16))) uint32_t act_s[kMaxChainGroup * (256 + 8)];  // r <= 256
  const int T = (a.V + 15) / 16, G = gridDim.x, w = blockIdx.x;
  const int t_begin = (int)((int64_t)T * w / G), t_end = (int)((int64_t)T * (w + 1) / G);
  act_clear_pads<W, KC>(act_s, a.B, a.r);  // made visible by the staging's barrier
  auto ready = [] { return true; };
  if (a.out_logits)
    logits_range_<W, RG, KC, true, false, decltype(ready), kSample>(a, p, t_begin, t_end, sbest, ready, 0u, act_s);
  else
    logits_range_<W, RG, KC, false, false, decltype(ready), kSample>(a, p, t_begin, t_end, sbest, ready, 0u, act_s);
}

// stepwise phase O with NWV waves per workgroup (one workgroup per CU)
template <class W, int RG, int KC, int NWV, bool kSample>
__global__ __launch_bounds__(64 * NWV) void chain_logits_wide_k(ChainArgs a, int p) {
  __shared__ uint64_t sbest[NWV * kMaxChainGroup];
  __shared__ __attribute__((aligned(16))) uint32_t act_s[kMaxChainGroup * (256 + 8)];  // r <= 256
  const int T = (a.V + 15) / 16, G = gridDim.x, w = blockIdx.x;
  const int t_begin = (int)((int64_t)T * w / G), t_end = (int)((int64_t)T * (w + 1) / G);
  act_clear_pads<W, KC>(act_s, a.B, a.r);  // made visible by the staging's barrier
  if (a.out_logits)
    logits_wide_<W, RG, KC, NWV, true, kSample>(a, p, t_begin, t_end, sbest, act_s);
  else
    logits_wide_<W, RG, KC, NWV, false, kSample>(a, p, t_begin, t_end, sbest, act_s);
}

// Stepwise schedule with phases W and O in one launch (bf16 weights): the
// first nW * ceil(B / 16) workgroups first compute one bottleneck item each
// (16 units of 16 sequences, NWV waves) and hand the activations out as
// tagged words of this call (tag: the call's epoch and p); then every
// workgroup stages those words and runs its vocabulary tiles, the item
// workgroups a smaller share of them.  The item workgroups have the lowest
// indices, so they are dispatched first and wait for no one: the launch
// needs no co-residency.  Waits are bounded (device status 2).
// sequences per bottleneck item of chain_wo_k: the state reads bound an item,
// so more items over fewer sequences each publish the activations sooner
// (batch 16, 8B shapes: 479 us per block with 16 sequences an item, 451 with 4)
constexpr int kWoSeqs = 4;
template <class W, int RG, int KC, int NWV, bool kSample>
__global__ __launch_bounds__(64 * NWV) void chain_wo_k(ChainArgs a, int p) {
  static_assert(sizeof(W) == 2, "bf16 weights");
  __shared__ uint64_t sbest[NWV * kMaxChainGroup];
  __shared__ __attribute__((aligned(16))) uint32_t act_s[kMaxChainGroup * (256 + 8)];  // r <= 256
  __shared__ __attribute__((aligned(16))) float red[16 * 64 * 4];                      // bottleneck chains
  const uint32_t ep = *a.epoch;  // advanced by the prologue launch of this call
  const int nW = (a.r + 15) / 16, nI = nW * ((a.B + kWoSeqs - 1) / kWoSeqs);
  const int T = (a.V + 15) / 16, G = gridDim.x, w = blockIdx.x;
  if (w < nI) {
    const int item = w % nW, seq0 = (w / nW) * kWoSeqs;
    bottleneck_item<W, 1, false, false, NWV, true>(a, p, item, red, nullptr, bottleneck_pre<1>(a, p, item, seq0), ep,
                                                   nullptr, seq0, seq0 + kWoSeqs);
  }
  int t_begin, t_end;
  o_tile_range(w, G, min(nI, G), T, t_begin, t_end);
  act_clear_pads<W, KC>(act_s, a.B, a.r);  // made visible by the staging's barrier
  if (a.out_logits)
    logits_wide_<W, RG, KC, NWV, true, kSample, true>(a, p, t_begin, t_end, sbest, act_s, ep);
  else
    logits_wide_<W, RG, KC, NWV, false, kSample, true>(a, p, t_begin, t_end, sbest, act_s, ep);
}

// All P steps in one launch (every workgroup resident); each owns one GRU work
// item (Hs/4 <= grid).  NTW == 0 (W2 streamed every step), kLds: 0 weights
// from global memory, 1 the GRU slice in LDS, 2 also the bottleneck slice of
// W1 in LDS.  NTW > 0 (W2 resident on chip): the GRU weights come from
// memory, W_ih fetched ahead of the token; kLds 2 puts the W1 slice in LDS;
// the LDS tier of W2 follows it.
template <class W, int RG, int KC, int kLds, int NTW, bool kTab, bool kSample>
__global__ __launch_bounds__(256) void chain_persistent(ChainArgs a) {
  static_assert(!kSample || NTW > 0, "sampling with W2 on chip only");
  constexpr int NCB = RG <= 2 ? 1 : 2;  // 16-sequence column blocks of phases G and W
  constexpr bool kGruLds = kLds >= 1 && NTW == 0;
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
  __shared__ __attribute__((aligned(16))) float red[4 * NCB * 64 * 4];
  __shared__ uint64_t sbest[4 * kMaxChainGroup];
  // dynamic LDS: [staged activations][GRU slice (streamed W2)][W1 slice][LDS
  // tier of W2 (resident W2)]
  uint32_t* act_s = reinterpret_cast<uint32_t*>(dyn_lds);
  act_clear_pads<W, KC>(act_s, a.B, a.r);  // made visible by the first staging's barrier
  W* gl = reinterpret_cast<W*>(dyn_lds + act_stage_bytes(a.B, KC, sizeof(W)));
  W* wl = gl + (kGruLds ? gru_slice_elems(a.d, a.Hs) : 0);
  const int G = gridDim.x, wg = blockIdx.x;
  const int nG = a.Hs / 4, nW = (a.r + 15) / 16, T = (a.V + 15) / 16;
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
  if (wg < nW && a.zh_splits > 1) zh_sum_rows(a, wg);
  // resident W2: the bottleneck workgroups stage the state words after their
  // LDS tiles when one poll round covers them (more rounds cost a memory
  // round trip each, more than per-lane polling)
  uint32_t* h_s = NTW > 0 && wg < nW && stage_state(a.B, a.Hs)
                      ? reinterpret_cast<uint32_t*>(w2l + (size_t)max(0, t_end - t_begin - 4 * NTW) * w2_lds_tile_bytes(KC))
                      : nullptr;
  f32x4 acc_h[4][NCB];  // hidden half of this workgroup's next GRU step, chains (wv, 0..3)
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc_h[j][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  __shared__ int32_t tok_s[kMaxChainGroup];
  __shared__ uint64_t sred_t[4 * kMaxChainGroup];
  const uint32_t ep = *a.epoch;  // advanced by the prologue launch
  float h_own = 0.f;             // this lane's own unit of the GRU state, h(0) = 0
  for (int p = 0; p < a.P; ++p) {
    if (wg == 0 && threadIdx.x == 0) a.stamps[p] = wall_clock64();
    // G: the previous token of every sequence, then one GRU step for this workgroup's units
    if (p > 0) ll_tokens_reduce(a, p - 1, ep, sred_t);
    BottleneckPre pre{};  // bottleneck terms known before the state: fetched during the GRU step
    if (wg < nG) {
      const int32_t* tk = nullptr;  // step 0 reads the first tokens
      if constexpr (NTW > 0) {
        // the token first: loads issued before its poll would delay it (wait
        // counts retire in order); W_ih then comes from L2 while the
        // embedding row comes from HBM
        if (p > 0) {
          ll_tokens_read(a, p - 1, ep, tok_s);
          tk = tok_s;
        }
        if (wg < nW) pre = bottleneck_pre<NCB, true>(a, p, wg);
        frag_t<W> xw[kXPre];
        if constexpr (!kTab) gru_x_prefetch<W>(a, wg, xw);
        DH_STAMP(p, 0);
        if (wg == 0 && p > 0)
          for (int b = threadIdx.x; b < a.B; b += blockDim.x) a.out_tokens[(size_t)b * a.P + p - 1] = tok_s[b];
        gru_finish_pre<W, NCB, kTab>(a, p, wg, red, xw, acc_h, tk, h_own, ep);
      } else {
        if (p > 0) {
          ll_tokens_read(a, p - 1, ep, tok_s);
          tk = tok_s;
        }
        if (wg < nW) pre = bottleneck_pre<NCB, true>(a, p, wg);
        DH_STAMP(p, 0);
        if (wg == 0 && p > 0)
          for (int b = threadIdx.x; b < a.B; b += blockDim.x) a.out_tokens[(size_t)b * a.P + p - 1] = tok_s[b];
        gru_finish<W, NCB, kGruLds, true, kTab>(a, p, wg, red, gl, acc_h, tk, &h_own, ep);
      }
    }
    DH_STAMP(p, 1);
    // W: the bottleneck of this step from h(p+1)
    if (wg < nW) {
      if (wg >= nG) pre = bottleneck_pre<NCB, true>(a, p, wg);
      DH_STAMP(p, 2);
      bottleneck_item<W, NCB, (kLds >= 2), true>(a, p, wg, red, wl, pre, ep, h_s);
    }
    DH_STAMP(p, 3);
    // W_hh h(p+1) for the next step: in the wait for the bottleneck, or, in
    // the bottleneck workgroups, after phase O
    const bool hidden = wg < nG && p + 1 < a.P;
    if (hidden && wg >= nW) gru_hidden_part<W, NCB, kGruLds, true>(a, p + 1, wg, gl, acc_h, ep);
    // O: this workgroup's vocabulary tiles, then its argmax pairs
    if constexpr (NTW > 0)
      logits_resident<W, RG, KC, NTW, kSample>(a, p, t_begin, t_end, w2r, w2l, act_s, sbest, ep);
    else
      logits_range<W, RG, KC, true>(a, p, t_begin, t_end, sbest, [] { return true; }, ep, act_s);
    DH_STAMP(p, 5);
    if (hidden && wg < nW) gru_hidden_part<W, NCB, kGruLds, true>(a, p + 1, wg, gl, acc_h, ep);
    DH_STAMP(p, 15);
  }
  ll_tokens_reduce(a, a.P - 1, ep, sred_t);
  if (wg == 0) {
    ll_tokens_read(a, a.P - 1, ep, tok_s);
    for (int b = threadIdx.x; b < a.B; b += blockDim.x) a.out_tokens[(size_t)b * a.P + a.P - 1] = tok_s[b];
    if (threadIdx.x == 0) a.stamps[a.P] = wall_clock64();
  }
}

// ---- host side ------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Splits of the H half's k range: enough workgroups in the prologue to
// spread its reads over about 256 CUs, at most kMaxZhSplits, at least four
// chunks of 32 per split.
int zh_splits(int d, int r, int P, int B) {
  const int tiles = ((r + 15) / 16) * ((B * P + 15) / 16), nck = (d + 31) / 32;
  int s = (256 + tiles - 1) / tiles;
  s = s < kMaxZhSplits ? s : kMaxZhSplits;
  s = s < nck / 4 ? s : nck / 4;
  return s > 1 ? s : 1;
}

ChainLayout chain_layout(int d, int Hs, int r, int P, int group) {
  ChainLayout L;
  size_t off = 0;
  L.status = off;
  off += 256;
  L.stamps = off;
  off += align256((size_t)(P + 1) * 8);
  L.keys = off;
  off += align256((size_t)P * group * 8);
  L.zh = off;
  size_t zh_floats = 0;  // the partials of any launch of up to `group` sequences
  for (int b = 1; b <= group; ++b) {
    const size_t f = (size_t)zh_splits(d, r, P, b) * b * P * r;
    zh_floats = f > zh_floats ? f : zh_floats;
  }
  off += align256(zh_floats * 4);
  L.zh_sum = off;
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
  L.ll_h = off;
  off += (size_t)(P + 1) * group * Hs * 8;
  L.ll_act = off;
  off += align256((size_t)P * group * r * 8);
  L.ll_part = off;
  off += (size_t)P * kMaxChainGrid * group * 16;
  L.ll_tok = off;
  off += align256((size_t)P * group * 16);
  L.trace = off;
#ifdef DH_TRACE_PHASES
  off += (size_t)P * 1024 * kTraceSlots * 8;
#endif
  L.total = off;
  return L;
}

// Dynamic LDS a resident-W2 launch on G workgroups needs (staged
// activations; in bottleneck workgroups the W1 slice; the LDS tiles; in
// bottleneck workgroups the staged state), or 0 if some workgroup owns more
// tiles than its register and LDS slots hold.
static size_t resident_lds(int G, const ChainArgs& a, int ntw, int kc, size_t w1_bytes) {
  const int nW = (a.r + 15) / 16, T = (a.V + 15) / 16;
  const size_t act = act_stage_bytes(a.B, kc, 2);  // resident W2 is bf16
  const size_t hst = stage_state(a.B, a.Hs) ? stage_words_bytes(a.B, a.Hs) : 0;  // staged state
  size_t need = act + w1_bytes + hst;
  for (int w = 0; w < G; ++w) {
    int b, e;
    o_tile_range(w, G, nW, T, b, e);
    const int n_lds = e - b - 4 * ntw;
    if (n_lds > kLdsTiles) return 0;
    const size_t at = act + (w < nW ? w1_bytes + hst : 0) + (size_t)(n_lds > 0 ? n_lds : 0) * w2_lds_tile_bytes(kc);
    need = at > need ? at : need;
  }
  return need;
}

struct CoopGrid {
  const void* fn = nullptr;
  int device = -1;
  size_t lds = 0;
  int blocks = 0;
};

// The persistent kernel needs all of its workgroups resident at the same
// time (they hand data to each other).  It is sized to one or two workgroups
// per CU and dispatched as an ordinary launch: a cooperative launch, which
// would guarantee residency, costs about 20 us of queue hand-over per call on
// this runtime.  Two persistent launches sharing the CUs could each wait for
// the other, so every persistent launch on a device first waits for the
// previous one, on whatever stream it ran.  Waits inside the kernel are
// bounded in any case (status 2).
struct PersistentGate {
  std::mutex m;
  hipEvent_t last = nullptr;
};
static PersistentGate g_gates[64];
static PersistentGate& persistent_gate(int dev) { return g_gates[dev & 63]; }

void release_chain_cache() {
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (int dev = 0; dev < 64; ++dev) {
    PersistentGate& g = g_gates[dev];
    std::lock_guard<std::mutex> lock(g.m);
    if (!g.last) continue;
    // the event belongs to device `dev`: wait for the last launch it marks, then free it
    if (hipSetDevice(dev) == hipSuccess) {
      (void)hipEventSynchronize(g.last);
      (void)hipEventDestroy(g.last);
    }
    g.last = nullptr;
  }
  if (have_cur) (void)hipSetDevice(cur);
}

template <class W, int RG, int KC, int kLds, int NTW, bool kTab, bool kSample>
static hipError_t launch_persistent_(const ChainArgs& a, size_t lds_bytes, hipStream_t s) {
  static thread_local CoopGrid cache;
  const void* fn = (const void*)chain_persistent<W, RG, KC, kLds, NTW, kTab, kSample>;
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
  if (cache.blocks > kMaxChainGrid || cache.blocks < a.B) return hipErrorInvalidConfiguration;  // hand-off slots
  // every workgroup must be resident at once: the grid is sized to what the
  // device holds, and launches are ordered per device (PersistentGate)
  PersistentGate& g = persistent_gate(dev);
  std::lock_guard<std::mutex> lock(g.m);
  if (g.last) {
    e = hipStreamWaitEvent(s, g.last, 0);
  } else {
    e = hipEventCreateWithFlags(&g.last, hipEventDisableTiming);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((chain_persistent<W, RG, KC, kLds, NTW, kTab, kSample>), dim3(cache.blocks), dim3(256), lds_bytes, s,
                     a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return hipEventRecord(g.last, s);
}
// with or without the per-token input table; sampled tokens (W2 on chip only)
template <class W, int RG, int KC, int kLds, int NTW, bool kSample = false>
static hipError_t launch_persistent(const ChainArgs& a, size_t lds_bytes, hipStream_t s) {
  return a.xt ? launch_persistent_<W, RG, KC, kLds, NTW, true, kSample>(a, lds_bytes, s)
              : launch_persistent_<W, RG, KC, kLds, NTW, false, kSample>(a, lds_bytes, s);
}

constexpr size_t kLdsBudget = 144 * 1024;  // dynamic LDS the persistent kernel may use (160 KB per CU)

template <class W, int RG, int KC>
static hipError_t run_chain(const ChainArgs& a, int mode, hipStream_t s, bool& persistent) {
  constexpr int NCB = RG <= 2 ? 1 : 2;
  const int cus = device_cus();
  // the persistent schedule needs one GRU work item per workgroup.  By
  // default it runs for up to 8 sequences (one row group), where the
  // hand-offs between its phases are what bounds a step; with more
  // sequences the three launches per step, each with all the waves a CU
  // holds for its phase, are faster.
  // fp32 weights (small models) always run the three launches per step;
  // sampling (temperature > 0) runs in one launch only with W2 on chip
  const bool sample = a.temperature > 0.f;
  persistent = sizeof(W) == 2 && (mode >= 2 || (mode == 0 && RG == 1)) && cus > 0 && a.Hs / 4 <= cus;
  if constexpr (sizeof(W) == 2) {
    if (persistent) {
      const size_t w = (size_t)16 * (a.Hs + 8) * sizeof(W);
      // W2 stays on chip (registers + LDS) when every workgroup's share fits;
      // the grid is then one workgroup per CU
      if constexpr (NCB == 1 && resident_fits<W, KC>()) {
        constexpr int NTW = resident_tiles<KC>();
        if (mode == 0 || mode == 3) {
          const size_t l2 = resident_lds(cus, a, NTW, KC, w);
          if (l2 > 0 && l2 <= kLdsBudget)
            return sample ? launch_persistent<W, RG, KC, 2, NTW, true>(a, l2, s)
                          : launch_persistent<W, RG, KC, 2, NTW, false>(a, l2, s);
        }
      }
    }
    if (persistent && sample) persistent = false;  // three launches per step
    if (persistent) {
      const size_t g = gru_slice_elems(a.d, a.Hs) * sizeof(W);
      const size_t w = (size_t)16 * (a.Hs + 8) * sizeof(W);
      const size_t act = act_stage_bytes(a.B, KC, sizeof(W));
      if (act + g + w <= kLdsBudget) return launch_persistent<W, RG, KC, 2, 0>(a, act + g + w, s);
      if (act + g <= kLdsBudget) return launch_persistent<W, RG, KC, 1, 0>(a, act + g, s);
      return launch_persistent<W, RG, KC, 0, 0>(a, act, s);
    }
  }
  const int nG = a.Hs / 4, nW = (a.r + 15) / 16, T = (a.V + 15) / 16;
  const int nO = T < cus ? T : (cus > 0 ? cus : 256);
  // phase G, bf16 weights: sixteen waves per work item
  const bool gru16 = sizeof(W) == 2;
  const bool tab = a.xt != nullptr;
  // the sixteen-wave GRU with the state staged in LDS (per-token table, more than 16
  // sequences, state within the LDS): 620 -> 605 us per block at 32 sequences, while
  // at 16 it measured slower (496 -> 505 us)
  const size_t lds16 = gru16_stage_bytes(a.B, a.Hs, NCB);
  bool stage16 = false;
  if constexpr (sizeof(W) == 2 && NCB == 2) {
    if (gru16 && tab && lds16 <= 144 * 1024) {
      stage16 = true;
      static thread_local int attr_dev = -1;
      int dev = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e != hipSuccess) return e;
      if (attr_dev != dev) {
        e = hipFuncSetAttribute((const void*)chain_gru16_k<W, NCB, true, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                144 * 1024);
        if (e != hipSuccess) return e;
        attr_dev = dev;
      }
    }
  }
  for (int p = 0; p < a.P; ++p) {
    if constexpr (sizeof(W) == 2) {
      if (gru16) {
        if (tab && stage16)
          hipLaunchKernelGGL((chain_gru16_k<W, NCB, true, true>), dim3(nG), dim3(1024), lds16, s, a, p);
        else if (tab)
          hipLaunchKernelGGL((chain_gru16_k<W, NCB, true>), dim3(nG), dim3(1024), 0, s, a, p);
        else
          hipLaunchKernelGGL((chain_gru16_k<W, NCB, false>), dim3(nG), dim3(1024), 0, s, a, p);
      } else if (tab) {
        hipLaunchKernelGGL((chain_gru_k<W, NCB, true>), dim3(nG), dim3(256), 0, s, a, p);
      } else {
        hipLaunchKernelGGL((chain_gru_k<W, NCB, false>), dim3(nG), dim3(256), 0, s, a, p);
      }
    } else if (tab) {
      hipLaunchKernelGGL((chain_gru_k<W, NCB, true>), dim3(nG), dim3(256), 0, s, a, p);
    } else {
      hipLaunchKernelGGL((chain_gru_k<W, NCB, false>), dim3(nG), dim3(256), 0, s, a, p);
    }
    constexpr int NWV = RG * KC >= 16 ? 8 : 16;  // waves per CU, as registers allow
    if constexpr (sizeof(W) == 2 && RG <= 2) {
      // bf16, up to 16 sequences: phase W inside the phase-O launch (measured
      // 453 -> 386 us per block at one sequence; at 32 sequences the 32 item
      // workgroups take as long as the separate launch, which stays)
      const int nI = nW * ((a.B + kWoSeqs - 1) / kWoSeqs), nWO = nO > nI ? nO : nI;
      if (sample)
        hipLaunchKernelGGL((chain_wo_k<W, RG, KC, NWV, true>), dim3(nWO), dim3(64 * NWV), 0, s, a, p);
      else
        hipLaunchKernelGGL((chain_wo_k<W, RG, KC, NWV, false>), dim3(nWO), dim3(64 * NWV), 0, s, a, p);
    } else if constexpr (sizeof(W) == 2) {  // bf16: many light waves per CU
      // one workgroup per 16 rows and 4 sequences (most of each MFMA's columns
      // left out): more CUs share the state reads, which bound this launch
      // (batch 32: 604 us per block with 16 sequences a workgroup, 593 with
      // 8, 587 with 4)
      hipLaunchKernelGGL((chain_bottleneck_k<W, 1>), dim3(nW, (a.B + 3) / 4), dim3(256), 0, s, a, p, 4);
      if (sample)
        hipLaunchKernelGGL((chain_logits_wide_k<W, RG, KC, NWV, true>), dim3(nO), dim3(64 * NWV), 0, s, a, p);
      else
        hipLaunchKernelGGL((chain_logits_wide_k<W, RG, KC, NWV, false>), dim3(nO), dim3(64 * NWV), 0, s, a, p);
    } else {
      // one workgroup per 16 rows and 16 sequences: more CUs share the state reads
      hipLaunchKernelGGL((chain_bottleneck_k<W, 1>), dim3(nW, (a.B + 15) / 16), dim3(256), 0, s, a, p, 16);
      if (sample)
        hipLaunchKernelGGL((chain_logits_k<W, RG, KC, true>), dim3(nO), dim3(256), 0, s, a, p);
      else
        hipLaunchKernelGGL((chain_logits_k<W, RG, KC, false>), dim3(nO), dim3(256), 0, s, a, p);
    }
  }
  return hipGetLastError();
}

// Phase O always runs 8 k chunks of 32 (r <= 256): chunks past r meet zero
// activations (the staged rows are zero padded) and add exact zeros, so a
// smaller rank gives the same values as a kernel sized for it.
template <class W, int RG>
static hipError_t run_chain_kc(const ChainArgs& a, int mode, hipStream_t s, bool& persistent) {
  if (a.r > 8 * 32) return hipErrorInvalidValue;
  return run_chain<W, RG, 8>(a, mode, s, persistent);
}

hipError_t launch_chain(int dtype, const ChainArgs& a, const void* H, int mode, bool reset_status, hipStream_t s,
                        hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (a.B <= 0) return hipSuccess;
  const dim3 pro((a.r + 15) / 16, (a.B * a.P + 15) / 16, a.zh_splits);
  if (dtype == kBF16)
    hipLaunchKernelGGL(chain_prologue<uint16_t>, pro, dim3(256), 0, s, a, H, reset_status ? 1 : 0);
  else
    hipLaunchKernelGGL(chain_prologue<float>, pro, dim3(256), 0, s, a, H, reset_status ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // row groups of 8 sequences in phase O
  const int rg = a.B <= 8 ? 1 : (a.B <= 16 ? 2 : 4);
  bool persistent = false;
  if (ev_start && ev_stop) {
    e = hipEventRecord(ev_start, s);
    if (e != hipSuccess) return e;
  }
  if (dtype == kBF16)
    e = rg == 1 ? run_chain_kc<uint16_t, 1>(a, mode, s, persistent)
                : (rg == 2 ? run_chain_kc<uint16_t, 2>(a, mode, s, persistent) : run_chain_kc<uint16_t, 4>(a, mode, s, persistent));
  else
    e = rg == 1 ? run_chain_kc<float, 1>(a, mode, s, persistent)
                : (rg == 2 ? run_chain_kc<float, 2>(a, mode, s, persistent) : run_chain_kc<float, 4>(a, mode, s, persistent));
  if (e != hipSuccess) return e;
  if (ev_start && ev_stop) {
    e = hipEventRecord(ev_stop, s);
    if (e != hipSuccess) return e;
  }
  if (!persistent) hipLaunchKernelGGL(chain_finalize, dim3((a.B * a.P + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dh
