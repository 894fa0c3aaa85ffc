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

__device__ __forceinline__ float bias_at(const float* b, int i) { return b ? b[i] : 0.f; }
__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + expf(-x)); }

__device__ __forceinline__ int32_t prev_token(const ChainArgs& a, int p, int b) {
  int32_t t = p == 0 ? a.t0[b]
                     : amax_index(__hip_atomic_load(&a.keys[(size_t)(p - 1) * a.B + b], __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT));
  return (t < 0 || t >= a.V) ? 0 : t;  // out-of-range first tokens are flagged by chain_init
}

// ---- phase G: one GRU step for 4 units and all sequences ------------------------
template <class W, int NCB>
__device__ void gru_item(const ChainArgs& a, int p, int item, float* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int d = a.d, Hs = a.Hs, B = a.B;
  const int j0 = item * 4;
  // left-operand row `row` = 4u + g:  g = 0 r, 1 z, 2 n (input half only), 3 n (hidden half only)
  const int u = row >> 2, g = row & 3;
  const bool has_x = g != 3, has_h = g != 2;
  const int gx = g < 3 ? g : 2, gh = g < 2 ? g : 2;
  const W* rx = (const W*)a.w_ih + ((size_t)gx * Hs + j0 + u) * d + kg * 8;
  const W* rh = (const W*)a.w_hh + ((size_t)gh * Hs + j0 + u) * Hs + kg * 8;
  const float* h_in = a.h + (size_t)(p & 1) * B * Hs;
  float* h_out = a.h + (size_t)((p + 1) & 1) * B * Hs;

  const W* xe[NCB];
  const float* hv[NCB];
  bool bok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int b = cb * 16 + row;
    bok[cb] = b < B;
    const int tok = bok[cb] ? prev_token(a, p, b) : 0;
    xe[cb] = (const W*)a.embed + (size_t)tok * d + kg * 8;
    hv[cb] = h_in + (size_t)(bok[cb] ? b : 0) * Hs + kg * 8;
  }

  f32x4 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // input half: E[prev] is stored exactly in W, one MFMA per chunk
  constexpr int U = 4;
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
  // hidden half: fp32 state as a hi + lo pair
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
      h_out[(size_t)b * Hs + j] = (1.f - zg) * ng + zg * h_in[(size_t)b * Hs + j];
    }
  }
  __syncthreads();
}

// ---- phase W: 16 bottleneck units, all sequences ----------------------------------
template <class W, int NCB>
__device__ void bottleneck_item(const ChainArgs& a, int p, int item, float* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int Hs = a.Hs, B = a.B, r = a.r;
  const int k0 = item * 16;
  const W* rw = (const W*)a.w1 + (size_t)min(k0 + row, r - 1) * (a.d + Hs) + a.d + kg * 8;
  const float* h_new = a.h + (size_t)((p + 1) & 1) * B * Hs;
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
  constexpr int U = 2;
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
    float pre[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 v = *reinterpret_cast<const float4*>(&red[((w * NCB + cb) * 64 + lane) * 4]);
      pre[0] += v.x;
      pre[1] += v.y;
      pre[2] += v.z;
      pre[3] += v.w;
    }
    const int b = cb * 16 + row;
    if (b < B) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = k0 + kg * 4 + i;
        if (k >= r) break;
        const float z = pre[i] + a.zh[((size_t)b * a.P + p) * r + k] + bias_at(a.b1, k);
        const float s = z / (1.f + expf(-z));
        if constexpr (sizeof(W) == 2) {
          uint16_t* hi = (uint16_t*)a.act;
          const uint16_t h16 = f2bf(s);
          hi[(size_t)b * r + k] = h16;
          hi[(size_t)B * r + (size_t)b * r + k] = f2bf(s - bf2f(h16));
        } else {
          ((float*)a.act)[(size_t)b * r + k] = s;
        }
      }
    }
  }
  __syncthreads();
}

// ---- phase O: W2 tiles [t_begin, t_end), base add, argmax ---------------------------
template <class W, int NCB, int KC>
__device__ void logits_range(const ChainArgs& a, int p, int t_begin, int t_end, uint64_t* sbest) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int B = a.B, r = a.r, V = a.V, P = a.P;
  const bool vec4 = (V & 3) == 0;

  // right operands: the bottleneck activations of every sequence, all of k
  typename act<W>::type bf[NCB][KC];
  size_t lrow[NCB];
  bool bok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int b = cb * 16 + row;
    bok[cb] = b < B;
    lrow[cb] = ((size_t)(bok[cb] ? b : 0) * P + p) * V;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int k = c * 32 + kg * 8;
      const bool ok = bok[cb] && k < r;
      if constexpr (sizeof(W) == 2) {
        const uint16_t* hi = (const uint16_t*)a.act + (size_t)b * r + k;
        bf[cb][c].hi = load8_or_zero(hi, ok);
        bf[cb][c].lo = load8_or_zero(hi + (size_t)B * r, ok);
      } else {
        bf[cb][c] = load8_or_zero((const float*)a.act + (size_t)b * r + k, ok);
      }
    }
  }

  uint64_t best[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) best[cb] = 0;

  const W* w2 = (const W*)a.w2;
  auto load_tile = [&](int t, frag_t<W>(&af)[KC]) {
    const W* wr = w2 + (size_t)min(t * 16 + row, V - 1) * r + kg * 8;
#pragma unroll
    for (int c = 0; c < KC; ++c) af[c] = load8_or_zero(wr + c * 32, c * 32 + kg * 8 < r);
  };

  int t = t_begin + wv;
  frag_t<W> cur[KC], nxt[KC];
  if (t < t_end) load_tile(t, cur);
  while (t < t_end) {
    const int tn = t + 4;
    if (tn < t_end) load_tile(tn, nxt);
    const int vv = t * 16 + kg * 4;  // this lane's 4 vocabulary rows
    float lb[NCB][4];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const float* src = a.Lb + lrow[cb] + vv;
      if (vec4 && vv + 3 < V) {
        const float4 q = *reinterpret_cast<const float4*>(src);
        lb[cb][0] = q.x;
        lb[cb][1] = q.y;
        lb[cb][2] = q.z;
        lb[cb][3] = q.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) lb[cb][i] = vv + i < V ? src[i] : 0.f;
      }
    }
    float bb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) bb[i] = (a.b2 && vv + i < V) ? a.b2[vv + i] : 0.f;

    f32x4 acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma(cur[c], bf[cb][c], acc[cb]);

#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      if (!bok[cb]) continue;
      float L[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        L[i] = lb[cb][i] + acc[cb][i] + bb[i];
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
#pragma unroll
    for (int c = 0; c < KC; ++c) cur[c] = nxt[c];
    t = tn;
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
}

// ---- kernels ------------------------------------------------------------------------
__global__ void chain_init(ChainArgs a, int reset_status) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x, stride = gridDim.x * blockDim.x;
  for (int i = tid; i < a.P * a.B; i += stride) a.keys[i] = 0;
  for (int i = tid; i < a.B * a.Hs; i += stride) a.h[i] = 0.f;
  if (tid < 4) a.counters[tid] = 0;
  if (tid == 0) {
    int32_t s = reset_status ? 0 : *a.status;
    for (int b = 0; b < a.B; ++b)
      if ((a.t0[b] < 0 || a.t0[b] >= a.V) && s == 0) s = 1;
    *a.status = s;
  }
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
  for (int it = blockIdx.x; it < a.Hs / 4; it += gridDim.x) gru_item<W, NCB>(a, p, it, red);
}

template <class W, int NCB>
__global__ __launch_bounds__(256) void chain_bottleneck_k(ChainArgs a, int p) {
  __shared__ __attribute__((aligned(16))) float red[4 * NCB * 64 * 4];
  for (int it = blockIdx.x; it < (a.r + 15) / 16; it += gridDim.x) bottleneck_item<W, NCB>(a, p, it, red);
}

template <class W, int NCB, int KC>
__global__ __launch_bounds__(256) void chain_logits_k(ChainArgs a, int p) {
  __shared__ uint64_t sbest[4 * NCB * 16];
  const int T = (a.V + 15) / 16, G = gridDim.x, w = blockIdx.x;
  logits_range<W, NCB, KC>(a, p, (int)((int64_t)T * w / G), (int)((int64_t)T * (w + 1) / G), sbest);
}

template <class W, int NCB, int KC>
__global__ __launch_bounds__(256) void chain_persistent(ChainArgs a) {
  __shared__ __attribute__((aligned(16))) float red[4 * NCB * 64 * 4];
  __shared__ uint64_t sbest[4 * NCB * 16];
  const int G = gridDim.x, wg = blockIdx.x;
  const int nG = a.Hs / 4, nW = (a.r + 15) / 16, T = (a.V + 15) / 16;
  uint32_t* cG = a.counters + 0;
  uint32_t* cW = a.counters + 1;
  uint32_t* cO = a.counters + 2;
  const int t_begin = (int)((int64_t)T * wg / G), t_end = (int)((int64_t)T * (wg + 1) / G);
  for (int p = 0; p < a.P; ++p) {
    if (wg < nG) {
      if (p > 0 && !wg_wait_geq(cO, (uint32_t)(p * G), a.status)) return;
      for (int it = wg; it < nG; it += G) gru_item<W, NCB>(a, p, it, red);
    }
    wg_arrive(cG);
    if (wg < nW) {
      if (!wg_wait_geq(cG, (uint32_t)((p + 1) * G), a.status)) return;
      for (int it = wg; it < nW; it += G) bottleneck_item<W, NCB>(a, p, it, red);
    }
    wg_arrive(cW);
    if (!wg_wait_geq(cW, (uint32_t)((p + 1) * G), a.status)) return;
    logits_range<W, NCB, KC>(a, p, t_begin, t_end, sbest);
    wg_arrive(cO);
  }
}

// ---- host side ------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

ChainLayout chain_layout(int d, int Hs, int r, int P, int group) {
  (void)d;
  ChainLayout L;
  size_t off = 0;
  L.status = off;
  L.counters = off + 64;
  off += 256;
  L.keys = off;
  off += align256((size_t)P * group * 8);
  L.zh = off;
  off += align256((size_t)group * P * r * 4);
  L.h = off;
  off += align256((size_t)2 * group * Hs * 4);
  L.act = off;
  off += align256((size_t)group * r * 4);
  L.total = off;
  return L;
}

struct CoopGrid {
  const void* fn = nullptr;
  int device = -1;
  int blocks = 0;
};

template <class W, int NCB, int KC>
static hipError_t run_chain(const ChainArgs& a, int mode, hipStream_t s) {
  if (mode == 0) {
    static thread_local CoopGrid cache;
    const void* fn = (const void*)chain_persistent<W, NCB, KC>;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (cache.fn != fn || cache.device != dev) {
      int per_cu = 0, cus = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0);
      if (e != hipSuccess) return e;
      e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      if (per_cu < 1) return hipErrorInvalidConfiguration;
      cache.fn = fn;
      cache.device = dev;
      cache.blocks = cus * (per_cu > 2 ? 2 : per_cu);
    }
    ChainArgs arg = a;
    void* params[] = {&arg};
    return hipLaunchCooperativeKernel(fn, dim3(cache.blocks), dim3(256), params, 0, s);
  }
  const int nG = a.Hs / 4, nW = (a.r + 15) / 16, T = (a.V + 15) / 16;
  const int nO = T < 1024 ? T : 1024;
  for (int p = 0; p < a.P; ++p) {
    hipLaunchKernelGGL((chain_gru_k<W, NCB>), dim3(nG), dim3(256), 0, s, a, p);
    hipLaunchKernelGGL((chain_bottleneck_k<W, NCB>), dim3(nW), dim3(256), 0, s, a, p);
    hipLaunchKernelGGL((chain_logits_k<W, NCB, KC>), dim3(nO), dim3(256), 0, s, a, p);
  }
  return hipGetLastError();
}

template <class W, int NCB>
static hipError_t run_chain_kc(const ChainArgs& a, int mode, hipStream_t s) {
  switch ((a.r + 31) / 32) {
    case 1: return run_chain<W, NCB, 1>(a, mode, s);
    case 2: return run_chain<W, NCB, 2>(a, mode, s);
    case 3: return run_chain<W, NCB, 3>(a, mode, s);
    case 4: return run_chain<W, NCB, 4>(a, mode, s);
    case 5: return run_chain<W, NCB, 5>(a, mode, s);
    case 6: return run_chain<W, NCB, 6>(a, mode, s);
    case 7: return run_chain<W, NCB, 7>(a, mode, s);
    case 8: return run_chain<W, NCB, 8>(a, mode, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_chain(int dtype, const ChainArgs& a, int mode, bool reset_status, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  const int n_init = a.B * a.Hs > a.P * a.B ? a.B * a.Hs : a.P * a.B;
  hipLaunchKernelGGL(chain_init, dim3((n_init + 255) / 256), dim3(256), 0, s, a, reset_status ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool two = a.B > 16;
  if (dtype == kBF16)
    e = two ? run_chain_kc<uint16_t, 2>(a, mode, s) : run_chain_kc<uint16_t, 1>(a, mode, s);
  else
    e = two ? run_chain_kc<float, 2>(a, mode, s) : run_chain_kc<float, 1>(a, mode, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chain_finalize, dim3((a.B * a.P + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dh
