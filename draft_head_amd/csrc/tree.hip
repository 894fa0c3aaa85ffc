// DominoTree-style best-first draft tree on gfx950 (DominoTree summary,
// gist.science Chinese page, technical abstract, "方法论 / 核心组件"):
//  * the children of a node are scored with that node's own GRU correction,
//    i.e. conditioned on the path, while the backbone states H are shared;
//  * every expansion is restricted to the top-M marginal candidates of its
//    depth, so W2 is touched on M columns only;
//  * nodes are popped from a max-heap keyed by cumulative path log-prob
//    (here: the log-softmax over the M corrected candidate logits).
// Scores, GRU states and the bottleneck are computed in fp64 so the tree
// structure does not depend on summation order.
//
// Kernels, in launch order for one call:
//  tree_topm        T1: top-M of each base-logit row, ordered (value desc,
//                   index asc); one workgroup per row, a single pass with a
//                   running threshold and an LDS buffer trimmed by a bitonic sort
//  tree_prologue    W1[:, :d] H for every position in fp64; empty heaps; the
//                   anchor as each sequence's first node to expand
//  per round (N rounds):
//   tree_gru        fp64 GRU step of each sequence's current node
//   tree_expand_pop push the node's M children, then pop the best entry
#include <math.h>

#include "device.h"
#include "internal.h"

namespace dh {

// ---- T1: top-M candidates per row ---------------------------------------------------
constexpr int kTopCap = 2048;  // LDS key buffer; M <= kTopCap / 2

__device__ __forceinline__ uint64_t cand_key(float v, uint32_t idx) { return amax_key(v, idx); }
__device__ __forceinline__ float key_value(uint64_t k) {
  uint32_t u = (uint32_t)(k >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

// descending bitonic sort of buf[0..kTopCap) by the whole workgroup
__device__ void bitonic_desc(uint64_t* buf) {
  for (int size = 2; size <= kTopCap; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < kTopCap / 2; i += blockDim.x) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t a = buf[lo], b = buf[hi];
        if ((a < b) == desc) {
          buf[lo] = b;
          buf[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(256) void tree_topm(const float* __restrict__ Lb, int V, int M, int32_t* cand_idx,
                                                 float* cand_val, int32_t* status, int reset_status) {
  __shared__ uint64_t buf[kTopCap];
  __shared__ int count;
  __shared__ uint64_t thresh;
  const int row = blockIdx.x;
  if (reset_status && row == 0 && threadIdx.x == 0) *status = 0;
  const float* x = Lb + (size_t)row * V;
  if (threadIdx.x == 0) {
    count = 0;
    thresh = 0;
  }
  for (int i = threadIdx.x; i < kTopCap; i += blockDim.x) buf[i] = 0;
  __syncthreads();
  // chunks of 1024 elements: at most 1024 appends per chunk, and the buffer is
  // trimmed to M whenever fewer than 1024 free slots remain
  for (int c0 = 0; c0 < V; c0 += 1024) {
    const uint64_t th = thresh;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int v = c0 + q * 256 + threadIdx.x;
      if (v < V) {
        const uint64_t k = cand_key(x[v], (uint32_t)v);
        if (k > th) buf[atomicAdd(&count, 1)] = k;
      }
    }
    __syncthreads();
    if (count > kTopCap - 1024) {
      bitonic_desc(buf);
      if (threadIdx.x == 0) {
        count = M;
        thresh = buf[M - 1];
      }
      __syncthreads();
      for (int i = M + threadIdx.x; i < kTopCap; i += blockDim.x) buf[i] = 0;
      __syncthreads();
    }
  }
  bitonic_desc(buf);
  for (int j = threadIdx.x; j < M; j += blockDim.x) {
    const uint64_t k = buf[j];
    cand_idx[(size_t)row * M + j] = amax_index(k);
    cand_val[(size_t)row * M + j] = key_value(k);
  }
}

// ---- per-sequence control state ---------------------------------------------------------
struct TreeCur {
  int32_t slot;         // state slot of the node being expanded (0 = anchor, k+1 = node k)
  int32_t parent_slot;  // its parent's state slot, -1 for the anchor (zero state)
  int32_t token;        // token the node reads into the GRU
  int32_t depth;        // its depth (anchor 0); children are scored on row `depth`
  int32_t expand;       // 1 when this round expands it
  int32_t node;         // its node index (-1 for the anchor)
  double score;         // its cumulative score
};

__device__ __forceinline__ double bf_or_f(const void* p, int dtype, size_t i) {
  return dtype == kBF16 ? (double)bf2f(((const uint16_t*)p)[i]) : (double)((const float*)p)[i];
}

// W1[:, :d] H[b][p] in fp64, one output per thread; empty heaps; anchors
__global__ __launch_bounds__(256) void tree_prologue(TreeArgs t) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int n = t.B * t.P * t.r;
  if (i < n) {
    const int k = i % t.r, row = i / t.r;  // row = b * P + p
    double s0 = 0, s1 = 0, s2 = 0, s3 = 0;
    const size_t w0 = (size_t)k * (t.d + t.Hs), h0 = (size_t)row * t.d;
    int j = 0;
    for (; j + 4 <= t.d; j += 4) {
      s0 += bf_or_f(t.w1, t.dtype, w0 + j) * bf_or_f(t.H, t.dtype, h0 + j);
      s1 += bf_or_f(t.w1, t.dtype, w0 + j + 1) * bf_or_f(t.H, t.dtype, h0 + j + 1);
      s2 += bf_or_f(t.w1, t.dtype, w0 + j + 2) * bf_or_f(t.H, t.dtype, h0 + j + 2);
      s3 += bf_or_f(t.w1, t.dtype, w0 + j + 3) * bf_or_f(t.H, t.dtype, h0 + j + 3);
    }
    for (; j < t.d; ++j) s0 += bf_or_f(t.w1, t.dtype, w0 + j) * bf_or_f(t.H, t.dtype, h0 + j);
    t.zh[i] = (s0 + s1) + (s2 + s3);
  }
  if (i < t.B) {
    t.heap_count[i] = 0;
    TreeCur c;
    int32_t t0 = t.t0[i];
    if (t0 < 0 || t0 >= t.V) {
      atomicMax(t.status, 1);
      t0 = 0;
    }
    c.slot = 0;
    c.parent_slot = -1;
    c.token = t0;
    c.depth = 0;
    c.expand = t.P > 0 ? 1 : 0;
    c.node = -1;
    c.score = 0.0;
    reinterpret_cast<TreeCur*>(t.cur)[i] = c;
  }
}

// ---- fp64 GRU step of each sequence's current node -----------------------------------------
// Workgroup = 4 GRU units, wave w = unit 4*blockIdx + w.  Lanes split k in
// runs of 8; 6 partial sums (gi_r, gi_z, gi_n, gh_r, gh_z, gh_n) per sequence
// are reduced across the wave, and lane b finishes sequence b.
constexpr int kTreeSeqs = 8;  // sequences per GRU pass

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__global__ __launch_bounds__(256) void tree_gru(TreeArgs t, int b0) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int j = blockIdx.x * 4 + wv;
  if (j >= t.Hs) return;
  const int d = t.d, Hs = t.Hs;
  const TreeCur* cur = reinterpret_cast<const TreeCur*>(t.cur);
  const int nb = min(kTreeSeqs, t.B - b0);
  double acc[kTreeSeqs][6];
#pragma unroll
  for (int s = 0; s < kTreeSeqs; ++s)
#pragma unroll
    for (int g = 0; g < 6; ++g) acc[s][g] = 0.0;
  // input half: x = E[token]
  for (int k0 = lane * 8; k0 < d; k0 += 512) {
    double w[3][8];
#pragma unroll
    for (int g = 0; g < 3; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) w[g][e] = bf_or_f(t.w_ih, t.dtype, ((size_t)g * Hs + j) * d + k0 + e);
#pragma unroll
    for (int s = 0; s < kTreeSeqs; ++s) {
      if (s >= nb) break;
      const TreeCur c = cur[b0 + s];
      if (!c.expand) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double x = bf_or_f(t.embed, t.dtype, (size_t)c.token * d + k0 + e);
#pragma unroll
        for (int g = 0; g < 3; ++g) acc[s][g] += w[g][e] * x;
      }
    }
  }
  // hidden half: the parent's state (zero for the anchor)
  for (int k0 = lane * 8; k0 < Hs; k0 += 512) {
    double w[3][8];
#pragma unroll
    for (int g = 0; g < 3; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) w[g][e] = bf_or_f(t.w_hh, t.dtype, ((size_t)g * Hs + j) * Hs + k0 + e);
#pragma unroll
    for (int s = 0; s < kTreeSeqs; ++s) {
      if (s >= nb) break;
      const TreeCur c = cur[b0 + s];
      if (!c.expand || c.parent_slot < 0) continue;
      const double* hp = t.states + ((size_t)(b0 + s) * (t.N + 1) + c.parent_slot) * Hs;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double h = hp[k0 + e];
#pragma unroll
        for (int g = 0; g < 3; ++g) acc[s][3 + g] += w[g][e] * h;
      }
    }
  }
#pragma unroll
  for (int s = 0; s < kTreeSeqs; ++s)
#pragma unroll
    for (int g = 0; g < 6; ++g) acc[s][g] = wave_sum(acc[s][g]);
  if (lane < nb) {
    const TreeCur c = cur[b0 + lane];
    if (c.expand) {
      double a6[6];
#pragma unroll
      for (int s = 0; s < kTreeSeqs; ++s)
        if (s == lane)
#pragma unroll
          for (int g = 0; g < 6; ++g) a6[g] = acc[s][g];
      auto bi = [&](int row) { return t.b_ih ? (double)t.b_ih[row] : 0.0; };
      auto bh = [&](int row) { return t.b_hh ? (double)t.b_hh[row] : 0.0; };
      const double r = 1.0 / (1.0 + exp(-(a6[0] + bi(j) + a6[3] + bh(j))));
      const double z = 1.0 / (1.0 + exp(-(a6[1] + bi(Hs + j) + a6[4] + bh(Hs + j))));
      const double nn = tanh(a6[2] + bi(2 * Hs + j) + r * (a6[5] + bh(2 * Hs + j)));
      const double hprev =
          c.parent_slot < 0 ? 0.0 : t.states[((size_t)(b0 + lane) * (t.N + 1) + c.parent_slot) * Hs + j];
      t.states[((size_t)(b0 + lane) * (t.N + 1) + c.slot) * Hs + j] = (1.0 - z) * nn + z * hprev;
    }
  }
}

// ---- score the current node's children, push them, pop the best entry ----------------------
__device__ __forceinline__ bool entry_before(double sa, int4 ma, double sb, int4 mb) {
  if (sa != sb) return sa > sb;
  if (ma.x != mb.x) return ma.x < mb.x;  // parent index
  return ma.y < mb.y;                    // candidate rank
}

__global__ __launch_bounds__(256) void tree_expand_pop(TreeArgs t, int k) {
  __shared__ double S[4096];   // the node's GRU state (Hs <= 4096)
  __shared__ double a[256];    // bottleneck (r <= 256)
  __shared__ double l[256];    // corrected candidate logits (M <= 256)
  __shared__ double red_s[256];
  __shared__ int red_i[256];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int Hs = t.Hs, r = t.r, M = t.M, P = t.P, V = t.V;
  TreeCur* curp = reinterpret_cast<TreeCur*>(t.cur) + b;
  const TreeCur c = *curp;
  double* hs = t.heap_score + (size_t)b * t.heap_cap;
  int4* hm = t.heap_meta + (size_t)b * t.heap_cap;
  int count = t.heap_count[b];

  if (c.expand) {
    const int delta = c.depth;
    const double* st = t.states + ((size_t)b * (t.N + 1) + c.slot) * Hs;
    for (int i = tid; i < Hs; i += blockDim.x) S[i] = st[i];
    __syncthreads();
    // a = SiLU(W1 [H_delta ; S] + b1): wave per row, lanes split the state half
    for (int row = wv; row < r; row += 4) {
      double s = 0.0;
      const size_t w0 = (size_t)row * (t.d + Hs) + t.d;
      for (int jj = lane; jj < Hs; jj += 64) s += bf_or_f(t.w1, t.dtype, w0 + jj) * S[jj];
      s = wave_sum(s);
      if (lane == 0) {
        const double z = s + t.zh[((size_t)b * P + delta) * r + row] + (t.b1 ? (double)t.b1[row] : 0.0);
        a[row] = z / (1.0 + exp(-z));
      }
    }
    __syncthreads();
    // corrected candidate logits on row delta
    const int32_t* cidx = t.cand_idx + ((size_t)b * P + delta) * M;
    const float* Lrow = t.Lb + ((size_t)b * P + delta) * V;
    for (int j = wv; j < M; j += 4) {
      const int v = cidx[j];
      double s = 0.0;
      for (int kk = lane; kk < r; kk += 64) s += bf_or_f(t.w2, t.dtype, (size_t)v * r + kk) * a[kk];
      s = wave_sum(s);
      if (lane == 0) l[j] = (double)Lrow[v] + (t.b2 ? (double)t.b2[v] : 0.0) + s;
    }
    __syncthreads();
    // log-sum-exp over the M candidates (one wave)
    if (wv == 0) {
      double mx = -INFINITY;
      for (int j = lane; j < M; j += 64) mx = fmax(mx, l[j]);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) mx = fmax(mx, __shfl_xor(mx, m));
      double se = 0.0;
      for (int j = lane; j < M; j += 64) se += exp(l[j] - mx);
      se = wave_sum(se);
      if (lane == 0) red_s[0] = mx + log(se);
    }
    __syncthreads();
    const double lse = red_s[0];
    for (int j = tid; j < M; j += blockDim.x) {
      hs[count + j] = c.score + (l[j] - lse);
      hm[count + j] = make_int4(c.node, j, cidx[j], delta + 1);
    }
    count += M;
    __syncthreads();
  }

  // pop: best entry under (score desc, parent asc, rank asc)
  int best = -1;
  double bs = 0.0;
  int4 bm = make_int4(0, 0, 0, 0);
  for (int i = tid; i < count; i += blockDim.x) {
    const double s = hs[i];
    const int4 m = hm[i];
    if (best < 0 || entry_before(s, m, bs, bm)) {
      best = i;
      bs = s;
      bm = m;
    }
  }
  red_i[tid] = best;
  red_s[tid] = bs;
  __syncthreads();
  for (int half = blockDim.x / 2; half > 0; half >>= 1) {
    if (tid < half) {
      const int o = red_i[tid + half];
      if (o >= 0) {
        const int me = red_i[tid];
        if (me < 0 || entry_before(red_s[tid + half], hm[o], red_s[tid], hm[me])) {
          red_i[tid] = o;
          red_s[tid] = red_s[tid + half];
        }
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    const size_t o = (size_t)b * t.N + k;
    const int bi = red_i[0];
    TreeCur n;
    n.expand = 0;
    n.slot = k + 1;
    n.parent_slot = -1;
    n.token = 0;
    n.depth = 0;
    n.node = k;
    n.score = 0.0;
    if (bi < 0) {
      t.out_parents[o] = -1;
      t.out_tokens[o] = -1;
      if (t.out_depth) t.out_depth[o] = 0;
      if (t.out_scores) t.out_scores[o] = -INFINITY;
    } else {
      const double s = hs[bi];
      const int4 m = hm[bi];
      t.out_parents[o] = m.x;
      t.out_tokens[o] = m.z;
      if (t.out_depth) t.out_depth[o] = m.w;
      if (t.out_scores) t.out_scores[o] = s;
      hs[bi] = hs[count - 1];
      hm[bi] = hm[count - 1];
      count -= 1;
      n.expand = (m.w < P && k + 1 < t.N) ? 1 : 0;
      n.parent_slot = m.x + 1;  // node index -> state slot; the anchor's slot is 0
      n.token = m.z;
      n.depth = m.w;
      n.score = s;
    }
    t.heap_count[b] = count;
    *curp = n;
  }
}

// ---- host side ------------------------------------------------------------------------------
static size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

TreeLayout tree_layout(int d, int Hs, int r, int P, int group, int N, int M) {
  (void)d;
  TreeLayout L;
  size_t off = 0;
  L.status = off;
  off += 256;
  L.cand_idx = off;
  off += al256((size_t)group * P * M * 4);
  L.cand_val = off;
  off += al256((size_t)group * P * M * 4);
  L.zh = off;
  off += al256((size_t)group * P * r * 8);
  L.states = off;
  off += al256((size_t)group * (N + 1) * Hs * 8);
  L.heap_cap = N * M;
  L.heap_score = off;
  off += al256((size_t)group * L.heap_cap * 8);
  L.heap_meta = off;
  off += al256((size_t)group * L.heap_cap * 16);
  L.heap_count = off;
  off += al256((size_t)group * 4);
  L.cur = off;
  off += al256((size_t)group * 32);
  L.total = off;
  return L;
}

hipError_t launch_topm(const float* Lb, int rows, int V, int M, int32_t* idx, float* val, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(tree_topm, dim3(rows), dim3(256), 0, s, Lb, V, M, idx, val, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_tree(const TreeArgs& t, bool reset_status, hipStream_t s) {
  if (t.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(tree_topm, dim3(t.B * t.P), dim3(256), 0, s, t.Lb, t.V, t.M, t.cand_idx, t.cand_val, t.status,
                     reset_status ? 1 : 0);
  const int n = t.B * t.P * t.r;
  hipLaunchKernelGGL(tree_prologue, dim3((n + 255) / 256), dim3(256), 0, s, t);
  for (int k = 0; k < t.N; ++k) {
    for (int b0 = 0; b0 < t.B; b0 += kTreeSeqs)
      hipLaunchKernelGGL(tree_gru, dim3((t.Hs + 3) / 4), dim3(256), 0, s, t, b0);
    hipLaunchKernelGGL(tree_expand_pop, dim3(t.B), dim3(256), 0, s, t, k);
  }
  return hipGetLastError();
}

}  // namespace dh
