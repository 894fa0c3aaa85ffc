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
//  topm_segment     T1: top-M of each segment of each base-logit row, ordered
//                   (value desc, index asc): a bound from the waves' maxima,
//                   then a bitonic sort of the keys at or above it (a single
//                   pass with a running threshold when too many pass)
//  tree_prep        in one launch: the row's top-M from its segment lists
//                   (topm_merge when T1 runs alone), W1[:, :d] H for every
//                   position on the fp64 matrix cores, the per-call set-up
//                   (empty heaps; the anchor as each sequence's first node)
//                   and, with bf16 weights, round 0's GRU step
//  bf16 weights, per round k one
//   tree_round      round k's bottleneck, its score and pop, and round k+1's
//                   GRU step, handing over through tagged words
//  fp32 weights, per round:
//   tree_gru        fp64 GRU step of each sequence's current node
//   tree_bottleneck fp64 a = SiLU(W1 [H ; S] + b1) of those nodes
//   tree_score_pop  score and push the node's M children, then pop the best entry
#include <math.h>

#include "device.h"
#include "internal.h"

namespace dh {

// ---- T1: top-M candidates per row ---------------------------------------------------
// Each row is split into kTopSegs segments; one workgroup per segment keeps the
// segment's top M, then one workgroup per row merges the segment lists.
constexpr int kTopCap = 2048;  // LDS key buffer; M <= kTopCap / kTopSegs
constexpr int kTopSegs = 8;
constexpr int kTopInFlight = 16;  // row reads in flight per thread in each pass of topm_segment

__device__ __forceinline__ float key_value(uint64_t k) {
  uint32_t u = (uint32_t)(k >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

// descending bitonic sort of buf[0..n) (n a power of two) by the whole workgroup
__device__ void bitonic_desc(uint64_t* buf, int n = kTopCap) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n / 2; i += blockDim.x) {
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

// Top M keys (value bits, inverted index; key 0 = none) of the elements
// [v_begin, v_end) of row x, into out[0..M), in a single pass: keys above the
// running threshold (the M-th best so far) are appended to an LDS buffer,
// which is sorted and cut back to M whenever fewer than 1024 slots remain.
// The fallback of topm_segment for inputs whose threshold estimate admits
// too many candidates.
__device__ void topm_scan_iterative(const float* __restrict__ x, int v_begin, int v_end, int M, uint64_t* buf,
                                    int* count, uint64_t* thresh, uint64_t* out) {
  __syncthreads();
  if (threadIdx.x == 0) {
    *count = 0;
    *thresh = 0;
  }
  for (int i = threadIdx.x; i < kTopCap; i += blockDim.x) buf[i] = 0;
  __syncthreads();
  for (int c0 = v_begin; c0 < v_end; c0 += 1024) {
    float cur[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int v = c0 + q * 256 + threadIdx.x;
      cur[q] = x[min(v, v_end - 1)];
    }
    const uint64_t th = *thresh;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int v = c0 + q * 256 + threadIdx.x;
      if (v < v_end) {
        const uint64_t k = amax_key(cur[q], (uint32_t)v);
        if (k > th) {
          // at most kTopCap - 1024 keys are kept between rounds and a round
          // appends at most 1024, so the bound only guards the invariant
          const int pos = atomicAdd(count, 1);
          if (pos < kTopCap) buf[pos] = k;
        }
      }
    }
    __syncthreads();
    // every thread takes the branch on the same snapshot of the count, and
    // no thread appends again before all have read it
    const int n_now = *count;
    __syncthreads();
    if (n_now > kTopCap - 1024) {
      bitonic_desc(buf);
      if (threadIdx.x == 0) {
        *count = M;
        *thresh = buf[M - 1];
      }
      __syncthreads();
      for (int i = M + threadIdx.x; i < kTopCap; i += blockDim.x) buf[i] = 0;
      __syncthreads();
    }
  }
  bitonic_desc(buf);
  for (int j = threadIdx.x; j < M; j += blockDim.x) out[j] = buf[j];
}

// Order-preserving 32-bit image of a value, the high word of amax_key before
// -0.0 is folded: -0.0 maps to 0x7FFFFFFF, +0.0 to 0x80000000 (topm_fold).
__device__ __forceinline__ uint32_t topm_image(float v) {
  const uint32_t u = __float_as_uint(v);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ uint32_t topm_fold(uint32_t img) { return img == 0x7FFFFFFFu ? 0x80000000u : img; }
// element e of a row through a 32-bit byte offset from the row's start
__device__ __forceinline__ float topm_at(const float* x, int e) {
  return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(x) + (uint32_t)e * 4u);
}

// Top M keys of one row segment, sorted, key 0 = none.  Two passes over the
// segment.  Pass 1: every thread takes one of its elements (its largest
// value image); within each wave the ceil(M/4)-th largest of these keys is
// reached by at least ceil(M/4) distinct elements, so the smallest of the
// four waves' values, tau, is reached by at least M elements and cannot
// exceed the segment's M-th key (for any choice of elements; the largest
// makes it tight).  Pass 2 collects every key >= tau (for typical data a few
// times M), which are then sorted; it compares value images first and forms
// the whole key only where the image can reach tau.  More candidates than
// the LDS buffer holds send the segment to topm_scan_iterative.
__global__ __launch_bounds__(256) void topm_segment(const float* __restrict__ Lb, int V, int M, uint64_t* seg_keys,
                                                    int32_t* status, int reset_status) {
  __shared__ uint64_t buf[kTopCap];
  __shared__ int count;
  __shared__ uint64_t thresh;
  __shared__ uint64_t wq[4];
  const int seg = blockIdx.x, row = blockIdx.y;
  if (reset_status && seg == 0 && row == 0 && threadIdx.x == 0) *status = 0;
  const int per = (V + kTopSegs - 1) / kTopSegs;
  const int v_begin = seg * per, v_end = min(V, v_begin + per);
  const float* x = Lb + (size_t)row * V;
  uint64_t* out = seg_keys + ((size_t)row * kTopSegs + seg) * M;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (v_end <= v_begin) {  // empty segment
    for (int j = threadIdx.x; j < M; j += blockDim.x) out[j] = 0;
    return;
  }
  // kTopInFlight reads in flight per thread; the last, partial, block of a
  // segment reads from clamped addresses
  auto load_block = [&](int v0, bool full, float (&f)[kTopInFlight]) {
    if (full) {
#pragma unroll
      for (int q = 0; q < kTopInFlight; ++q) f[q] = topm_at(x, v0 + q * 256 + (int)threadIdx.x);
    } else {
#pragma unroll
      for (int q = 0; q < kTopInFlight; ++q) f[q] = topm_at(x, min(v0 + q * 256 + (int)threadIdx.x, v_end - 1));
    }
  };
  // pass 1
  uint32_t bu = 0;
  int bi = -1;
  for (int v0 = v_begin; v0 < v_end; v0 += kTopInFlight * 256) {
    const bool full = v0 + kTopInFlight * 256 <= v_end;
    float f[kTopInFlight];
    load_block(v0, full, f);
#pragma unroll
    for (int q = 0; q < kTopInFlight; ++q) {
      const int v = v0 + q * 256 + threadIdx.x;
      const uint32_t u = topm_image(f[q]);
      if ((full || v < v_end) && u > bu) {
        bu = u;
        bi = v;
      }
    }
  }
  uint64_t mk = bi < 0 ? 0 : ((uint64_t)topm_fold(bu) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)bi);
  // descending bitonic sort of the 64 maxima across the wave
  for (int size = 2; size <= 64; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint64_t o = shfl_xor_u64(mk, stride);
      const bool keep_max = ((lane & stride) == 0) == ((lane & size) == 0);
      mk = keep_max ? umax64(mk, o) : (mk < o ? mk : o);
    }
  const int qm = (M + 3) / 4;  // <= 64
  const uint64_t wk = ((uint64_t)__shfl((uint32_t)(mk >> 32), qm - 1) << 32) | __shfl((uint32_t)mk, qm - 1);
  if (lane == 0) wq[wv] = wk;
  if (threadIdx.x == 0) count = 0;
  __syncthreads();
  uint64_t tau = wq[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) tau = wq[w] < tau ? wq[w] : tau;
  // pass 2: every key >= tau.  A key reaches tau only if its folded image
  // reaches tau's high word tu, that is, only if the unfolded image reaches tu2.
  const uint32_t tu = (uint32_t)(tau >> 32), tu2 = tu == 0x80000000u ? 0x7FFFFFFFu : tu;
  for (int v0 = v_begin; v0 < v_end; v0 += kTopInFlight * 256) {
    const bool full = v0 + kTopInFlight * 256 <= v_end;
    float f[kTopInFlight];
    load_block(v0, full, f);
#pragma unroll
    for (int q = 0; q < kTopInFlight; ++q) {
      const int v = v0 + q * 256 + threadIdx.x;
      const uint32_t u = topm_image(f[q]);
      if ((full || v < v_end) && u >= tu2) {
        const uint64_t k = ((uint64_t)topm_fold(u) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)v);
        if (k >= tau && k != 0) {
          const int pos = atomicAdd(&count, 1);
          if (pos < kTopCap) buf[pos] = k;
        }
      }
    }
  }
  __syncthreads();
  const int n = count;
  if (n > kTopCap) {
    topm_scan_iterative(x, v_begin, v_end, M, buf, &count, &thresh, out);
    return;
  }
  int p2 = 64;
  while (p2 < n || p2 < M) p2 <<= 1;
  for (int i = n + threadIdx.x; i < p2; i += blockDim.x) buf[i] = 0;
  __syncthreads();
  bitonic_desc(buf, p2);
  for (int j = threadIdx.x; j < M; j += blockDim.x) out[j] = buf[j];
}

// merge the segment lists of one row into its top M
__device__ __forceinline__ void merge_row(const uint64_t* seg_keys, int M, int32_t* cand_idx, float* cand_val,
                                          int row) {
  __shared__ uint64_t buf[kTopCap];
  const uint64_t* src = seg_keys + (size_t)row * kTopSegs * M;
  int n = 64;  // the segment lists, padded to a power of two
  while (n < kTopSegs * M) n <<= 1;
  for (int i = threadIdx.x; i < n; i += blockDim.x) buf[i] = i < kTopSegs * M ? src[i] : 0;
  __syncthreads();
  bitonic_desc(buf, n);
  for (int j = threadIdx.x; j < M; j += blockDim.x) {
    const uint64_t k = buf[j];
    cand_idx[(size_t)row * M + j] = amax_index(k);
    cand_val[(size_t)row * M + j] = key_value(k);
  }
}
__global__ __launch_bounds__(256) void topm_merge(const uint64_t* seg_keys, int M, int32_t* cand_idx, float* cand_val) {
  merge_row(seg_keys, M, cand_idx, cand_val, blockIdx.x);
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

// Two cursor slots: round k reads slot k & 1 and its pop writes the other,
// so nothing that reads round k's cursor can see round k + 1's.
__device__ __forceinline__ TreeCur* tree_cur(const TreeArgs& t, int k) {
  return reinterpret_cast<TreeCur*>(t.cur) + (size_t)(k & 1) * t.B;
}

// ---- reductions across the 64 lanes of a wave, without LDS ---------------------------------
// The lanes of each row of 16 combine through DPP moves (swaps within quads,
// then the mirrored halves of the row, then the mirrored row); the four row
// results are read as uniform values and combined as (row 0 . row 1) .
// (row 2 . row 3).  The operation is commutative and each step pairs lanes
// symmetrically, so every lane ends with the same bits.
template <int kCtrl>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_mov_dpp(v, kCtrl, 0xF, 0xF, false);
}
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp_i32<kCtrl>((int)b), hi = dpp_i32<kCtrl>((int)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, l), hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowHalfMirror = 0x141, kDppRowMirror = 0x140;
template <class Op>
__device__ __forceinline__ double wave_reduce(double v, Op op) {
  v = op(v, dpp_f64<kDppQuadXor1>(v));
  v = op(v, dpp_f64<kDppQuadXor2>(v));
  v = op(v, dpp_f64<kDppRowHalfMirror>(v));
  v = op(v, dpp_f64<kDppRowMirror>(v));
  return op(op(readlane_f64(v, 0), readlane_f64(v, 16)), op(readlane_f64(v, 32), readlane_f64(v, 48)));
}
__device__ __forceinline__ double wave_sum(double v) {
  return wave_reduce(v, [](double x, double y) { return x + y; });
}
__device__ __forceinline__ double wave_max(double v) {
  return wave_reduce(v, [](double x, double y) { return fmax(x, y); });
}

// 8 consecutive stored elements widened to fp64
__device__ __forceinline__ void load8_f64(const void* base, int dtype, size_t i, double (&o)[8]) {
  if (dtype == kBF16) {
    const uint4 q = *reinterpret_cast<const uint4*>((const uint16_t*)base + i);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = (double)__uint_as_float(w[e] << 16);
      o[2 * e + 1] = (double)__uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else {
    const float4* q = reinterpret_cast<const float4*>((const float*)base + i);
    const float4 a = q[0], b = q[1];
    o[0] = a.x, o[1] = a.y, o[2] = a.z, o[3] = a.w, o[4] = b.x, o[5] = b.y, o[6] = b.z, o[7] = b.w;
  }
}

__device__ __forceinline__ void bf16x8_to_f64(const uint4& r, double (&o)[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[2 * e] = (double)__uint_as_float(w[e] << 16);
    o[2 * e + 1] = (double)__uint_as_float(w[e] & 0xFFFF0000u);
  }
}

struct F64x8 {
  double v[8];
};

__device__ __forceinline__ F64x8 load_f64x8(const double* p) {
  F64x8 r;
  const double4* q = reinterpret_cast<const double4*>(p);
  const double4 a = q[0], b = q[1];
  r.v[0] = a.x, r.v[1] = a.y, r.v[2] = a.z, r.v[3] = a.w;
  r.v[4] = b.x, r.v[5] = b.y, r.v[6] = b.z, r.v[7] = b.w;
  return r;
}

// eight consecutive weights of one row, as stored, and their fp64 values
template <class W>
struct Run8;
template <>
struct Run8<uint16_t> {
  uint4 u;
  __device__ void load(const uint16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ void get(double (&o)[8]) const { bf16x8_to_f64(u, o); }
};
template <>
struct Run8<float> {
  float4 a, b;
  __device__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ void get(double (&o)[8]) const {
    o[0] = a.x, o[1] = a.y, o[2] = a.z, o[3] = a.w, o[4] = b.x, o[5] = b.y, o[6] = b.z, o[7] = b.w;
  }
};

typedef double f64x4 __attribute__((ext_vector_type(4)));

// W1[:, :d] H[b][p] in fp64 for every (sequence, position) row, on the fp64
// matrix cores.  Workgroup = one 16 x 16 output tile: MFMA rows are 16 rows of
// W1 (bottleneck units), columns 16 rows of H.  The k range (d) runs in
// 32-wide blocks dealt to the 8 waves in turn; in a block, lane l holds 8
// consecutive k values, 8 (l / 16) + 0..7, of its row and column, and MFMA i
// takes value i of every lane.  The first kZhPre blocks of every wave are read
// before the first MFMA; the waves' sums meet in LDS in wave order.
constexpr int kZhWaves = 8, kZhPre = 10;

template <class W>
__device__ __forceinline__ void zh_tile(const TreeArgs& t, int kx, int my) {
  __shared__ double red[kZhWaves][4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rr = lane & 15, kq = lane >> 4;
  const int k0 = kx * 16, m0 = my * 16;
  const int d = t.d, r = t.r, rows = t.B * t.P;
  const W* wrow = reinterpret_cast<const W*>(t.w1) + (size_t)min(k0 + rr, r - 1) * ((size_t)d + t.Hs);
  const W* hrow = reinterpret_cast<const W*>(t.H) + (size_t)min(m0 + rr, rows - 1) * d;
  Run8<W> wa[kZhPre], ha[kZhPre];
#pragma unroll
  for (int q = 0; q < kZhPre; ++q) {
    const int j = min((wv + kZhWaves * q) * 32 + 8 * kq, d - 8);
    wa[q].load(wrow + j);
    ha[q].load(hrow + j);
  }
  __builtin_amdgcn_sched_barrier(0);
  f64x4 acc[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
#pragma unroll
  for (int q = 0; q < kZhPre; ++q) {
    const bool ok = (wv + kZhWaves * q) * 32 + 8 * kq < d;
    double w8[8], h8[8];
    wa[q].get(w8);
    ha[q].get(h8);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc[q & 1] = __builtin_amdgcn_mfma_f64_16x16x4f64(w8[i], ok ? h8[i] : 0.0, acc[q & 1], 0, 0, 0);
  }
  const int nbk = (d + 31) / 32;
  for (int bk = wv + kZhWaves * kZhPre; bk < nbk; bk += kZhWaves * 4) {  // wider H rows
    Run8<W> wb[4], hb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = min((bk + kZhWaves * q) * 32 + 8 * kq, d - 8);
      wb[q].load(wrow + j);
      hb[q].load(hrow + j);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool ok = (bk + kZhWaves * q) * 32 + 8 * kq < d;
      double w8[8], h8[8];
      wb[q].get(w8);
      hb[q].get(h8);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[q & 1] = __builtin_amdgcn_mfma_f64_16x16x4f64(w8[i], ok ? h8[i] : 0.0, acc[q & 1], 0, 0, 0);
    }
  }
  // result layout of the fp64 MFMA: register i of lane l holds row 4 i + l / 16 of column l % 16
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wv][i][lane] = acc[0][i] + acc[1][i];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int i = threadIdx.x >> 6, l = threadIdx.x & 63;
    double v = red[0][i][l];
#pragma unroll
    for (int w = 1; w < kZhWaves; ++w) v += red[w][i][l];
    const int k = k0 + 4 * i + (l >> 4), m = m0 + (l & 15);
    if (k < r && m < rows) t.zh[(size_t)m * r + k] = v;
  }
}

// empty heaps; the anchor as each sequence's first node to expand (one
// workgroup).  It also advances the call counter that tags the hand-off words
// of the one-launch-per-round schedule, after clearing those words on the
// first use of this workspace layout (or before the counter would overflow
// the tags).
__device__ __forceinline__ void tree_init(const TreeArgs& t) {
  {
    __shared__ int fresh;
    __shared__ uint32_t epoch_in;
    if (threadIdx.x == 0) {
      const uint64_t mk = *t.marker, sg = *t.sig;
      const uint32_t ep = *t.epoch;
      fresh = mk != kLLMarker || sg != t.sig_value || ep + 1 >= kEpochLimit;
      epoch_in = ep;
    }
    __syncthreads();
    if (fresh) {
      uint4* w = reinterpret_cast<uint4*>(t.ll_act);
      for (size_t i = threadIdx.x; i < t.ll_words / 2; i += blockDim.x) w[i] = make_uint4(0, 0, 0, 0);
      if (threadIdx.x == 0) {
        *t.marker = kLLMarker;
        *t.sig = t.sig_value;
      }
    }
    if (threadIdx.x == 0) *t.epoch = (fresh ? 0u : epoch_in) + 1u;
  }
  for (int b = threadIdx.x; b < t.B; b += blockDim.x) {
    t.heap_count[b] = 0;
    int32_t t0 = t.t0[b];
    if (t0 < 0 || t0 >= t.V) {
      atomicMax(t.status, 1);
      t0 = 0;
    }
    TreeCur c;
    c.slot = 0;
    c.parent_slot = -1;
    c.token = t0;
    c.depth = 0;
    c.expand = t.P > 0 ? 1 : 0;
    c.node = -1;
    c.score = 0.0;
    tree_cur(t, 0)[b] = c;
  }
}

// the node round 0 expands: the anchor, read from the first tokens (so that
// round 0's GRU step need not wait for tree_init)
__device__ __forceinline__ TreeCur anchor_cur(const TreeArgs& t, int b) {
  TreeCur c;
  c.slot = 0;
  c.parent_slot = -1;
  const int32_t t0 = t.t0[b];
  c.token = t0 < 0 || t0 >= t.V ? 0 : t0;  // as tree_init reads it (which also flags it)
  c.depth = 0;
  c.expand = t.P > 0 ? 1 : 0;
  c.node = -1;
  c.score = 0.0;
  return c;
}

// ---- fp64 GRU step of each sequence's current node -----------------------------------------
// Workgroup = 4 GRU units and 16 waves: wave w takes unit 4*blockIdx + w % 4
// for a quarter of the sequences (w / 4 selects which), so a SIMD runs four
// waves.
// The current nodes' embedding rows (stored type) and parent states (fp64) of
// up to kTreeSeqs sequences are staged in LDS; lanes split k in runs of 8 and
// the 6 partial sums (gi_r, gi_z, gi_n, gh_r, gh_z, gh_n) per sequence are
// reduced across the wave; lane s finishes the wave's sequence s.
constexpr int kTreeSeqs = 8;
constexpr int kSeqPerWave = 2;  // four waves per GRU unit, each with a quarter of the sequences

__global__ __launch_bounds__(1024) void tree_gru(TreeArgs t, int b0, int k) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ TreeCur sc[kTreeSeqs];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int d = t.d, Hs = t.Hs;
  const int es = t.dtype == kBF16 ? 2 : 4;
  const int nb = min(kTreeSeqs, t.B - b0);
  double* hl = reinterpret_cast<double*>(lds);                      // [kTreeSeqs][Hs]
  unsigned char* xl = lds + (size_t)kTreeSeqs * Hs * sizeof(double);  // [kTreeSeqs][d] stored type
  if (threadIdx.x < nb) sc[threadIdx.x] = tree_cur(t, k)[b0 + threadIdx.x];
  __syncthreads();
  // stage every sequence's parent state and embedding row: batches of kStage
  // 16-byte pieces per thread are loaded before any is stored, so their
  // latencies overlap (a load-store loop would pay one round trip per piece)
  {
    constexpr int kStage = 8;
    const int hchunks = Hs / 2, xchunks = d * es / 16;  // 16-byte pieces
    const int per = hchunks + xchunks, n = nb * per;
    auto src_of = [&](int i) -> const uint4* {
      const int s = i / per, q = i - s * per;
      const TreeCur& c = sc[s];
      if (q < hchunks) {
        // a node with no parent state reads slot 0 of its own sequence (zeros are stored instead)
        const int slot = c.parent_slot >= 0 ? c.parent_slot : 0;
        return reinterpret_cast<const uint4*>(t.states + ((size_t)(b0 + s) * (t.N + 1) + slot) * Hs) + q;
      }
      return reinterpret_cast<const uint4*>((const unsigned char*)t.embed + (size_t)c.token * d * es) + (q - hchunks);
    };
    auto dst_of = [&](int i) -> uint4* {
      const int s = i / per, q = i - s * per;
      if (q < hchunks) return reinterpret_cast<uint4*>(hl + (size_t)s * Hs) + q;
      return reinterpret_cast<uint4*>(xl + (size_t)s * d * es) + (q - hchunks);
    };
    for (int base = 0; base < n; base += kStage * (int)blockDim.x) {
      uint4 v[kStage];
#pragma unroll
      for (int k = 0; k < kStage; ++k) {
        const int i = base + k * (int)blockDim.x + threadIdx.x;
        v[k] = i < n ? *src_of(i) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < kStage; ++k) {
        const int i = base + k * (int)blockDim.x + threadIdx.x;
        if (i < n) {
          const int s = i / per, q = i - s * per;
          const TreeCur& c = sc[s];
          const bool zero = q < hchunks && !(c.expand && c.parent_slot >= 0);
          *dst_of(i) = zero ? make_uint4(0, 0, 0, 0) : v[k];
        }
      }
    }
  }
  __syncthreads();
  // wave wv: unit blockIdx * 4 + wv % 4, sequences s0 .. s0 + kSeqPerWave - 1
  const int j = blockIdx.x * 4 + (wv & 3), s0 = (wv >> 2) * kSeqPerWave;  // waves 4q .. 4q+3: quarter q
  if (j >= Hs) return;
  int expand[kSeqPerWave];
#pragma unroll
  for (int s = 0; s < kSeqPerWave; ++s) expand[s] = s0 + s < nb ? sc[s0 + s].expand : 0;
  double acc[kSeqPerWave][6];
#pragma unroll
  for (int s = 0; s < kSeqPerWave; ++s)
#pragma unroll
    for (int g = 0; g < 6; ++g) acc[s][g] = 0.0;
  // input half, R 8-wide runs of every gate row in flight at a time (read
  // from the per-token table instead when there is one)
  constexpr int R = 1;
  for (int k0 = lane * 8; k0 < (t.xt ? 0 : d); k0 += 512 * R) {
    double w[R][3][8];
#pragma unroll
    for (int u = 0; u < R; ++u)
#pragma unroll
      for (int g = 0; g < 3; ++g)
        if (k0 + u * 512 < d) load8_f64(t.w_ih, t.dtype, ((size_t)g * Hs + j) * d + k0 + u * 512, w[u][g]);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      if (k0 + u * 512 >= d) break;
#pragma unroll
      for (int s = 0; s < kSeqPerWave; ++s) {
        if (!expand[s]) continue;
        double x[8];
        load8_f64(xl + (size_t)(s0 + s) * d * es, t.dtype, k0 + u * 512, x);
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int g = 0; g < 3; ++g) acc[s][g] += w[u][g][e] * x[e];
      }
    }
  }
  for (int k0 = lane * 8; k0 < Hs; k0 += 512 * R) {
    double w[R][3][8];
#pragma unroll
    for (int u = 0; u < R; ++u)
#pragma unroll
      for (int g = 0; g < 3; ++g)
        if (k0 + u * 512 < Hs) load8_f64(t.w_hh, t.dtype, ((size_t)g * Hs + j) * Hs + k0 + u * 512, w[u][g]);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      if (k0 + u * 512 >= Hs) break;
#pragma unroll
      for (int s = 0; s < kSeqPerWave; ++s) {
        if (!expand[s]) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double h = hl[(size_t)(s0 + s) * Hs + k0 + u * 512 + e];
#pragma unroll
          for (int g = 0; g < 3; ++g) acc[s][3 + g] += w[u][g][e] * h;
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < kSeqPerWave; ++s)
#pragma unroll
    for (int g = 0; g < 6; ++g) acc[s][g] = wave_sum(acc[s][g]);
  double a6[6] = {0, 0, 0, 0, 0, 0};
  int mine = 0;
#pragma unroll
  for (int s = 0; s < kSeqPerWave; ++s)
    if (s == lane) {
      mine = expand[s];
#pragma unroll
      for (int g = 0; g < 6; ++g) a6[g] = acc[s][g];
    }
  const int sq = s0 + lane;  // the sequence this lane finishes
  if (lane < kSeqPerWave && sq < nb && mine) {
    const TreeCur c = sc[sq];
    if (t.xt) {
      const double* q = t.xt + (size_t)min(max(c.token, 0), t.V - 1) * 3 * Hs + j;
      a6[0] = q[0];
      a6[1] = q[Hs];
      a6[2] = q[2 * Hs];
    }
    auto bi = [&](int row) { return t.b_ih ? (double)t.b_ih[row] : 0.0; };
    auto bh = [&](int row) { return t.b_hh ? (double)t.b_hh[row] : 0.0; };
    const double r = 1.0 / (1.0 + exp(-(a6[0] + bi(j) + a6[3] + bh(j))));
    const double z = 1.0 / (1.0 + exp(-(a6[1] + bi(Hs + j) + a6[4] + bh(Hs + j))));
    const double nn = tanh(a6[2] + bi(2 * Hs + j) + r * (a6[5] + bh(2 * Hs + j)));
    const double hprev = hl[(size_t)sq * Hs + j];
    t.states[((size_t)(b0 + sq) * (t.N + 1) + c.slot) * Hs + j] = (1.0 - z) * nn + z * hprev;
  }
}

// ---- per-token input half in fp64: table[v][g] = sum_k embed[v][k] w_ih[g][k] ----------------
// Workgroup = a 64 x 64 block of the table (64 tokens, 64 gate rows), four
// waves in 2 x 2, each four 16 x 16 fp64 MFMA tiles (rows: tokens, columns:
// gate rows).  k runs in 32-wide blocks; in a block lane l holds 8 consecutive
// k values, 8 (l / 16) + 0..7, of its token row and of its gate row, and MFMA
// i takes value i of every lane (the products are exact in fp64).  Loads go
// straight from memory into registers; rows past the end repeat the last
// row and are not stored, k past d contributes zeros.
template <class W>
__global__ __launch_bounds__(256) void input_table_f64_k(const W* __restrict__ E, const W* __restrict__ Wih, int V,
                                                         int G3, int d, double* __restrict__ table) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rr = lane & 15, kq = lane >> 4;
  const int t0 = blockIdx.x * 64 + (wv >> 1) * 32, g0 = blockIdx.y * 64 + (wv & 1) * 32;
  const W* er[2];
  const W* wr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    er[i] = E + (size_t)min(t0 + 16 * i + rr, V - 1) * d;
    wr[i] = Wih + (size_t)min(g0 + 16 * i + rr, G3 - 1) * d;
  }
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int k0 = 0; k0 < d; k0 += 32) {
    const int k = k0 + 8 * kq;
    const bool ok = k < d;  // d is a multiple of 8: a lane's run is all in or all out
    const int kc = ok ? k : 0;
    Run8<W> ra[2], rb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ra[i].load(er[i] + kc);
      rb[i].load(wr[i] + kc);
    }
    double a8[2][8], b8[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ra[i].get(a8[i]);
      rb[i].get(b8[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) a8[i][e] = ok ? a8[i][e] : 0.0;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a8[i][e], b8[j][e], acc[i][j], 0, 0, 0);
  }
  // register q of lane l holds row 4 q + l / 16 (token) of column l % 16 (gate row)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + 16 * i + 4 * q + kq, g = g0 + 16 * j + rr;
        if (t < V && g < G3) table[(size_t)t * G3 + g] = acc[i][j][q];
      }
}

hipError_t launch_input_table_f64(int dtype, const void* E, const void* Wih, int V, int Hs, int d, double* table,
                                  hipStream_t s) {
  const int G3 = 3 * Hs;
  const dim3 grid((V + 63) / 64, (G3 + 63) / 64);
  if (dtype == kBF16)
    hipLaunchKernelGGL(input_table_f64_k<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)E, (const uint16_t*)Wih, V,
                       G3, d, table);
  else
    hipLaunchKernelGGL(input_table_f64_k<float>, grid, dim3(256), 0, s, (const float*)E, (const float*)Wih, V, G3, d,
                       table);
  return hipGetLastError();
}

// ---- the same GRU step on the fp64 matrix cores (bf16 weights) ----------------------------
// Workgroup = 4 GRU units.  The MFMA's 16 rows are the r, z and n rows of
// those units (rows 12..15 repeat row 11; their results are not used) and its
// 16 columns the sequences (columns past the last repeat it, unused).  The k
// range runs in 32-wide blocks dealt to the 8 waves in turn; in a block, lane
// l holds 8 consecutive k values, 8 (l / 16) + 0..7, of its row and column,
// and MFMA i of the block takes value i of every lane, so the 8 MFMAs cover
// the block's 32 k values (4 each).  Each lane reads its own operands (weight
// row, embedding row or parent state of its column) straight from memory:
// nothing is staged, so the matrix cores start as soon as the first block
// lands and the only barrier is the one before the cross-wave sum.  The
// input half (W_ih E[token]) and the hidden half (W_hh h) have their own
// accumulators; the waves' partial sums meet in LDS, in wave order, and 32
// threads finish (unit, sequence) pairs.




constexpr int kGruWaves = 8;  // waves of a GRU-step workgroup (bf16 weights), splitting the k blocks
constexpr int kGruPreI = 10;  // input-half blocks per wave whose loads are all issued up front
constexpr int kGruPreH = 4;   // hidden-half blocks per wave whose loads are all issued up front

// kTab: the input half comes from the per-token fp64 table (t.xt) instead.
// kLL (one launch per round): the node of round kr arrives as the hand-off
// words of round kr - 1's pop (tag), polled by wave 0 while the weight loads
// are in flight; otherwise it is read from round kr's cursor.
template <bool kTab, bool kLL>
__device__ __forceinline__ void gru_mfma_step(const TreeArgs& t, int b0, int item, int kr, uint32_t tag) {
  __shared__ double red[kGruWaves][2][12][kTreeSeqs];  // [wave][input, hidden][gate row][sequence]
  __shared__ int cur_s[kTreeSeqs][3];                   // kLL: token, parent slot, expand
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int d = t.d, Hs = t.Hs;
  const int nb = min(kTreeSeqs, t.B - b0);
  const int j0 = item * 4;
  const int rr = lane & 15, kq = lane >> 4;  // A row and B column; k group
  const int g = rr < 12 ? rr >> 2 : 2, u = rr < 12 ? rr & 3 : 3;
  const size_t wrow = (size_t)g * Hs + min(j0 + u, Hs - 1);
  const uint16_t* wi = (const uint16_t*)t.w_ih + wrow * d;
  const uint16_t* wh = (const uint16_t*)t.w_hh + wrow * Hs;
  // the weights do not depend on the tree: their loads go out first
  uint4 wpi[kGruPreI], wph[kGruPreH];
  if constexpr (!kTab) {
#pragma unroll
    for (int q = 0; q < kGruPreI; ++q)
      wpi[q] = *reinterpret_cast<const uint4*>(wi + min((wv + kGruWaves * q) * 32 + 8 * kq, d - 8));
  }
#pragma unroll
  for (int q = 0; q < kGruPreH; ++q)
    wph[q] = *reinterpret_cast<const uint4*>(wh + min((wv + kGruWaves * q) * 32 + 8 * kq, Hs - 8));
  // this lane's column: sequence sq's token row and parent state (zeros without a parent)
  const int sq = min(rr, nb - 1);
  TreeCur c;
  if constexpr (kLL) {
    if (wv == 0) {
      const uint64_t* src = t.ll_cur + ((size_t)(kr - 1) * t.B + b0 + min(lane, nb - 1)) * 2;
      uint64_t w0 = 0, w1 = 0;
      ll_wait(t.status, [&] {
        w0 = ld_agent64(src);
        w1 = ld_agent64(src + 1);
        return (int)ll_ok(w0, tag) & (int)ll_ok(w1, tag);
      });
      if (lane < nb) {  // (clamped, so that words left by a timed-out wait stay in bounds)
        const uint32_t v = ll_data(w1);
        cur_s[lane][0] = (int)ll_data(w0);
        cur_s[lane][1] = (int)min(v & 0xFFFFu, (uint32_t)kr) - 1;
        cur_s[lane][2] = (int)((v >> 16) & 1u);
      }
    }
    __syncthreads();
    c.slot = kr;
    c.token = cur_s[sq][0];
    c.parent_slot = cur_s[sq][1];
    c.expand = cur_s[sq][2];
    c.depth = 0;
    c.node = kr - 1;
    c.score = 0.0;
  } else {
    c = kr == 0 ? anchor_cur(t, b0 + sq) : tree_cur(t, kr)[b0 + sq];
  }
  const bool has_h = c.expand && c.parent_slot >= 0;
  const uint16_t* xr = (const uint16_t*)t.embed + (size_t)min(max(c.token, 0), t.V - 1) * d;
  const double* hr = t.states + ((size_t)(b0 + sq) * (t.N + 1) + max(c.parent_slot, 0)) * Hs;
  // the finishing lanes (wave 0, lanes 0..31: unit lane / 8, sequence lane % 8)
  // take their sequence's cursor from lane lane % 8, whose column it is
  const int fs = lane & 7, fu = (lane >> 3) & 3;
  const int f_slot = __shfl(c.slot, fs), f_ps = __shfl(c.parent_slot, fs);
  const int f_exp = __shfl(c.expand, fs);
  uint4 xp[kGruPreI];
  double gx[3] = {0.0, 0.0, 0.0};  // kTab: the finishing lane's input half from the table
  if constexpr (kTab) {
    const int f_tok = __shfl(c.token, fs);
    if (threadIdx.x < 4 * kTreeSeqs) {
      const double* q = t.xt + (size_t)min(max(f_tok, 0), t.V - 1) * 3 * Hs + min(j0 + fu, Hs - 1);
      gx[0] = q[0];
      gx[1] = q[Hs];
      gx[2] = q[2 * Hs];
    }
  } else {
#pragma unroll
    for (int q = 0; q < kGruPreI; ++q)
      xp[q] = *reinterpret_cast<const uint4*>(xr + min((wv + kGruWaves * q) * 32 + 8 * kq, d - 8));
  }
  F64x8 hp[kGruPreH];
#pragma unroll
  for (int q = 0; q < kGruPreH; ++q) hp[q] = load_f64x8(hr + min((wv + kGruWaves * q) * 32 + 8 * kq, Hs - 8));
  const double hprev_raw =
      t.states[((size_t)(b0 + min(fs, nb - 1)) * (t.N + 1) + max(f_ps, 0)) * Hs + min(j0 + fu, Hs - 1)];
  // every load above is issued before the first MFMA (the scheduler would
  // otherwise move them next to their uses and wait on each in turn)
  __builtin_amdgcn_sched_barrier(0);

  // two accumulators per half (even and odd blocks), summed at the end
  f64x4 acc_i[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
  f64x4 acc_h[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
#pragma unroll
  for (int q = 0; q < (kTab ? 0 : kGruPreI); ++q) {
    const bool ok = (wv + kGruWaves * q) * 32 + 8 * kq < d;
    double w8[8], x8[8];
    bf16x8_to_f64(wpi[q], w8);
    bf16x8_to_f64(xp[q], x8);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc_i[q & 1] = __builtin_amdgcn_mfma_f64_16x16x4f64(w8[i], ok ? x8[i] : 0.0, acc_i[q & 1], 0, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < kGruPreH; ++q) {
    const bool ok = has_h && (wv + kGruWaves * q) * 32 + 8 * kq < Hs;
    double w8[8];
    bf16x8_to_f64(wph[q], w8);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc_h[q & 1] = __builtin_amdgcn_mfma_f64_16x16x4f64(w8[i], ok ? hp[q].v[i] : 0.0, acc_h[q & 1], 0, 0, 0);
  }
  // blocks past those (wider hidden sizes), four in flight at a time
  constexpr int NB = 4;
  const int nbi = kTab ? 0 : (d + 31) / 32, nbh = (Hs + 31) / 32;
  for (int bk = wv + kGruWaves * kGruPreI; bk < nbi; bk += kGruWaves * NB) {
    uint4 wr[NB], xv[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int k = min((bk + kGruWaves * q) * 32 + 8 * kq, d - 8);
      wr[q] = *reinterpret_cast<const uint4*>(wi + k);
      xv[q] = *reinterpret_cast<const uint4*>(xr + k);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const bool ok = (bk + kGruWaves * q) * 32 + 8 * kq < d;
      double w8[8], x8[8];
      bf16x8_to_f64(wr[q], w8);
      bf16x8_to_f64(xv[q], x8);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc_i[q & 1] = __builtin_amdgcn_mfma_f64_16x16x4f64(w8[i], ok ? x8[i] : 0.0, acc_i[q & 1], 0, 0, 0);
    }
  }
  for (int bk = wv + kGruWaves * kGruPreH; bk < nbh; bk += kGruWaves * NB) {
    uint4 wr[NB];
    F64x8 hv[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int k = min((bk + kGruWaves * q) * 32 + 8 * kq, Hs - 8);
      wr[q] = *reinterpret_cast<const uint4*>(wh + k);
      hv[q] = load_f64x8(hr + k);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const bool ok = has_h && (bk + kGruWaves * q) * 32 + 8 * kq < Hs;
      double w8[8];
      bf16x8_to_f64(wr[q], w8);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc_h[q & 1] = __builtin_amdgcn_mfma_f64_16x16x4f64(w8[i], ok ? hv[q].v[i] : 0.0, acc_h[q & 1], 0, 0, 0);
    }
  }
  // result layout of the fp64 MFMA: register i of lane l holds row 4 i + l / 16 of column l % 16
  if (rr < kTreeSeqs) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {  // rows 12..15 (i = 3) are padding
      red[wv][0][4 * i + kq][rr] = acc_i[0][i] + acc_i[1][i];
      red[wv][1][4 * i + kq][rr] = acc_h[0][i] + acc_h[1][i];
    }
  }
  __syncthreads();
  if (threadIdx.x < 4 * kTreeSeqs) {
    const int j = j0 + fu;
    if (fs < nb && j < Hs && f_exp) {
      double gi[3], gh[3];
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        gi[q] = red[0][0][4 * q + fu][fs];
        gh[q] = red[0][1][4 * q + fu][fs];
#pragma unroll
        for (int w = 1; w < kGruWaves; ++w) {
          gi[q] += red[w][0][4 * q + fu][fs];
          gh[q] += red[w][1][4 * q + fu][fs];
        }
        if constexpr (kTab) gi[q] = gx[q];
      }
      auto bi = [&](int row) { return t.b_ih ? (double)t.b_ih[row] : 0.0; };
      auto bh = [&](int row) { return t.b_hh ? (double)t.b_hh[row] : 0.0; };
      const double r = 1.0 / (1.0 + exp(-(gi[0] + bi(j) + gh[0] + bh(j))));
      const double z = 1.0 / (1.0 + exp(-(gi[1] + bi(Hs + j) + gh[1] + bh(Hs + j))));
      const double nn = tanh(gi[2] + bi(2 * Hs + j) + r * (gh[2] + bh(2 * Hs + j)));
      const double hprev = f_ps >= 0 ? hprev_raw : 0.0;
      t.states[((size_t)(b0 + fs) * (t.N + 1) + f_slot) * Hs + j] = (1.0 - z) * nn + z * hprev;
    }
  }
}

// The GRU step of round kr in the one-launch-per-round schedule with the
// per-token table.  The hidden half does not depend on which node is popped:
// before the node arrives, the workgroup multiplies its units' W_hh rows by
// the state of slot kr - 1 (written by the previous launch) for every
// sequence of the group, the same MFMA blocks and wave order as
// gru_mfma_step, and keeps the sums in t.gh, where every later round finds the
// hidden half of any parent.  Once the node arrives, its finishing lanes read
// the parent's hidden half, the table row of its token and the parent's own
// units of the state, and apply the gates: the result has the bits of
// gru_mfma_step's.
__device__ __forceinline__ void gru_tab_ll_step(const TreeArgs& t, int b0, int item, int kr, uint32_t tag) {
  __shared__ double red[kGruWaves][12][kTreeSeqs];  // [wave][gate row][sequence], hidden half
  __shared__ int cur_s[kTreeSeqs][3];               // token, parent slot, expand
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int Hs = t.Hs;
  const int nb = min(kTreeSeqs, t.B - b0);
  const int j0 = item * 4;
  const int rr = lane & 15, kq = lane >> 4;
  const int g = rr < 12 ? rr >> 2 : 2, u = rr < 12 ? rr & 3 : 3;
  const uint16_t* wh = (const uint16_t*)t.w_hh + ((size_t)g * Hs + min(j0 + u, Hs - 1)) * Hs;
  const int sq = min(rr, nb - 1);
  const int ps = kr - 1;  // the slot whose hidden half this launch adds to t.gh
  // Start once the bottleneck of the group's first sequence is out (when that
  // node is expanded): the state reads below would otherwise share the memory
  // system with the bottleneck's hand-off, which is on the round's critical
  // path, while this work has until the popped node arrives (286 against
  // 298 us per tree at batch 8).  A matter of timing only: nothing read here
  // depends on it.
  if (threadIdx.x == 0 && tree_cur(t, kr - 1)[b0].expand) {
    const uint64_t* w = t.ll_act + (((size_t)(kr - 1) * t.B + b0) * t.r + t.r - 1) * 2;
    ll_wait<4>(t.status, [&] { return (int)ll_ok(ld_agent64(w), tag); });
  }
  __syncthreads();
  const double* hr = t.states + ((size_t)(b0 + sq) * (t.N + 1) + ps) * Hs;
  uint4 wph[kGruPreH];
  F64x8 hp[kGruPreH];
#pragma unroll
  for (int q = 0; q < kGruPreH; ++q) {
    const int k = min((wv + kGruWaves * q) * 32 + 8 * kq, Hs - 8);
    wph[q] = *reinterpret_cast<const uint4*>(wh + k);
    hp[q] = load_f64x8(hr + k);
  }
  __builtin_amdgcn_sched_barrier(0);
  f64x4 acc_h[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
#pragma unroll
  for (int q = 0; q < kGruPreH; ++q) {
    const bool ok = (wv + kGruWaves * q) * 32 + 8 * kq < Hs;
    double w8[8];
    bf16x8_to_f64(wph[q], w8);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc_h[q & 1] = __builtin_amdgcn_mfma_f64_16x16x4f64(w8[i], ok ? hp[q].v[i] : 0.0, acc_h[q & 1], 0, 0, 0);
  }
  constexpr int NB = 4;
  const int nbh = (Hs + 31) / 32;
  for (int bk = wv + kGruWaves * kGruPreH; bk < nbh; bk += kGruWaves * NB) {  // wider states
    uint4 wr[NB];
    F64x8 hv[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int k = min((bk + kGruWaves * q) * 32 + 8 * kq, Hs - 8);
      wr[q] = *reinterpret_cast<const uint4*>(wh + k);
      hv[q] = load_f64x8(hr + k);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const bool ok = (bk + kGruWaves * q) * 32 + 8 * kq < Hs;
      double w8[8];
      bf16x8_to_f64(wr[q], w8);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc_h[q & 1] = __builtin_amdgcn_mfma_f64_16x16x4f64(w8[i], ok ? hv[q].v[i] : 0.0, acc_h[q & 1], 0, 0, 0);
    }
  }
  if (rr < kTreeSeqs) {
#pragma unroll
    for (int i = 0; i < 3; ++i) red[wv][4 * i + kq][rr] = acc_h[0][i] + acc_h[1][i];
  }
  __syncthreads();
  const int fs = lane & 7, fu = (lane >> 3) & 3, j = j0 + fu;
  const bool fin = threadIdx.x < 4 * kTreeSeqs && fs < nb && j < Hs;
  double* ghp = t.gh + (size_t)(b0 + fs) * (t.N + 1) * 3 * Hs + j;
  if (fin) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      double v = red[0][4 * q + fu][fs];
#pragma unroll
      for (int w = 1; w < kGruWaves; ++w) v += red[w][4 * q + fu][fs];
      ghp[((size_t)ps * 3 + q) * Hs] = v;
    }
  }
  // the node of round kr: the hand-off words of round kr - 1's pop
  if (wv == 0) {
    const uint64_t* src = t.ll_cur + ((size_t)(kr - 1) * t.B + b0 + min(lane, nb - 1)) * 2;
    uint64_t w0 = 0, w1 = 0;
    ll_wait(t.status, [&] {
      w0 = ld_agent64(src);
      w1 = ld_agent64(src + 1);
      return (int)ll_ok(w0, tag) & (int)ll_ok(w1, tag);
    });
    if (lane < nb) {  // (clamped, so that words left by a timed-out wait stay in bounds)
      const uint32_t v = ll_data(w1);
      cur_s[lane][0] = (int)ll_data(w0);
      cur_s[lane][1] = (int)min(v & 0xFFFFu, (uint32_t)kr) - 1;
      cur_s[lane][2] = (int)((v >> 16) & 1u);
    }
  }
  __syncthreads();
  if (fin && cur_s[fs][2]) {
    const int tok = min(max(cur_s[fs][0], 0), t.V - 1), par = cur_s[fs][1];
    const double* q = t.xt + (size_t)tok * 3 * Hs + j;
    double gi[3] = {q[0], q[Hs], q[2 * Hs]}, gh[3] = {0.0, 0.0, 0.0};
    double hprev = 0.0;
    if (par >= 0) {
#pragma unroll
      for (int i = 0; i < 3; ++i) gh[i] = ghp[((size_t)par * 3 + i) * Hs];
      hprev = t.states[((size_t)(b0 + fs) * (t.N + 1) + par) * Hs + j];
    }
    auto bi = [&](int row) { return t.b_ih ? (double)t.b_ih[row] : 0.0; };
    auto bh = [&](int row) { return t.b_hh ? (double)t.b_hh[row] : 0.0; };
    const double r = 1.0 / (1.0 + exp(-(gi[0] + bi(j) + gh[0] + bh(j))));
    const double z = 1.0 / (1.0 + exp(-(gi[1] + bi(Hs + j) + gh[1] + bh(Hs + j))));
    const double nn = tanh(gi[2] + bi(2 * Hs + j) + r * (gh[2] + bh(2 * Hs + j)));
    t.states[((size_t)(b0 + fs) * (t.N + 1) + kr) * Hs + j] = (1.0 - z) * nn + z * hprev;
  }
}



// ---- fp64 bottleneck of each sequence's current node: a = SiLU(W1 [H_delta ; S] + b1) -------
// Rows k0 .. k0 + 3 of sequence b's bottleneck in round kr, by one wave whose
// lanes split the state.
// kLL: the results go out as hand-off words of round kr (tag), else to t.act.
template <class W, bool kLL>
__device__ __forceinline__ void bottleneck_rows(const TreeArgs& t, int b, int k0, int kr, uint32_t tag) {
  constexpr int U = 2;  // runs of 8 per lane and row whose reads go out first (state width <= 1024)
  const int lane = threadIdx.x & 63;
  const int Hs = t.Hs, r = t.r;
  const size_t ld = (size_t)t.d + Hs;
  const W* w1s = reinterpret_cast<const W*>(t.w1) + t.d;  // state half of W1
  // Nothing here reads the cursor: the node expanded in round kr has state
  // slot kr, and the previous pop left the H half of its depth in zh_cur
  // (round 0: the anchor, depth 0).  A sequence whose node is not expanded gets values that no
  // one reads.
  Run8<W> wr[U][4];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q) wr[u][q].load(w1s + (size_t)min(k0 + q, r - 1) * ld + min(lane * 8 + 512 * u, Hs - 8));
  const double* st = t.states + ((size_t)b * (t.N + 1) + kr) * Hs;
  F64x8 sv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) sv[u] = load_f64x8(st + min(lane * 8 + 512 * u, Hs - 8));
  // lane q < 4 finishes row k0 + q: its W1_H half and bias
  const int kq = min(k0 + (lane & 3), r - 1);
  const double zq = kr == 0 ? t.zh[(size_t)b * t.P * r + kq] : t.zh_cur[(size_t)b * r + kq];
  const double bq = t.b1 ? (double)t.b1[kq] : 0.0;
  __builtin_amdgcn_sched_barrier(0);
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (lane * 8 + 512 * u >= Hs) break;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      double w[8];
      wr[u][q].get(w);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[q] += w[e] * sv[u].v[e];
    }
  }
  for (int jj = lane * 8 + 512 * U; jj < Hs; jj += 512) {  // wider states
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      Run8<W> x;
      x.load(w1s + (size_t)min(k0 + q, r - 1) * ld + jj);
      double w[8];
      x.get(w);
      const F64x8 sx = load_f64x8(st + jj);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[q] += w[e] * sx.v[e];
    }
  }
  double v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = wave_sum(acc[q]);
  const int k = k0 + lane;
  if (lane < 4 && k < r) {
    const double z = (lane == 0 ? v[0] : lane == 1 ? v[1] : lane == 2 ? v[2] : v[3]) + zq + bq;
    const double a = z / (1.0 + exp(-z));
    if constexpr (kLL) {
      const uint64_t bits = (uint64_t)__double_as_longlong(a);
      uint64_t* w = t.ll_act + (((size_t)kr * t.B + b) * r + k) * 2;
      ll_put(w, (uint32_t)bits, tag);
      ll_put(w + 1, (uint32_t)(bits >> 32), tag);
    } else {
      t.act[(size_t)b * r + k] = a;
    }
  }
}

// Workgroup = 16 bottleneck rows of one sequence, four per wave.
template <class W>
__global__ __launch_bounds__(256) void tree_bottleneck(TreeArgs t, int k) {
  bottleneck_rows<W, false>(t, blockIdx.y, blockIdx.x * 16 + (threadIdx.x >> 6) * 4, k, 0u);
}

// ---- score the current node's children, push them, pop the best entry ----------------------
// Heap order: higher score first, then lower parent index, then lower
// candidate rank.  The running best of a scan is kept without branches: the
// comparison is evaluated with bitwise logic and every field is replaced
// through a select.  The empty state (score -inf, parent and rank INT_MAX) loses to any real entry.  A
// divergent `if (first || before) { copy the whole entry }` was compiled into
// code that kept the old token and depth on one of the two paths into the
// copy, so the form below is used wherever the entry's meta is consumed.
struct BestEntry {
  int slot;
  double s;
  int4 m;
};

__device__ __forceinline__ BestEntry best_empty() {
  BestEntry e;
  e.slot = -1;
  e.s = -INFINITY;
  e.m = make_int4(INT_MAX, INT_MAX, 0, 0);
  return e;
}

__device__ __forceinline__ void best_offer(BestEntry& e, int slot, double s, int4 m, bool valid = true) {
  const bool take = valid & ((s > e.s) | ((s == e.s) & ((m.x < e.m.x) | ((m.x == e.m.x) & (m.y < e.m.y)))));
  e.slot = take ? slot : e.slot;
  e.s = take ? s : e.s;
  e.m.x = take ? m.x : e.m.x;
  e.m.y = take ? m.y : e.m.y;
  e.m.z = take ? m.z : e.m.z;
  e.m.w = take ? m.w : e.m.w;
}

// the best entry of the wave, in every lane (the same pairing as wave_reduce;
// the order is total over distinct entries, so the result is symmetric)
template <int kCtrl>
__device__ __forceinline__ void best_offer_dpp(BestEntry& e) {
  best_offer(e, dpp_i32<kCtrl>(e.slot), dpp_f64<kCtrl>(e.s),
             make_int4(dpp_i32<kCtrl>(e.m.x), dpp_i32<kCtrl>(e.m.y), dpp_i32<kCtrl>(e.m.z), dpp_i32<kCtrl>(e.m.w)));
}
__device__ __forceinline__ BestEntry best_readlane(const BestEntry& e, int l) {
  BestEntry o;
  o.slot = __builtin_amdgcn_readlane(e.slot, l);
  o.s = readlane_f64(e.s, l);
  o.m = make_int4(__builtin_amdgcn_readlane(e.m.x, l), __builtin_amdgcn_readlane(e.m.y, l),
                  __builtin_amdgcn_readlane(e.m.z, l), __builtin_amdgcn_readlane(e.m.w, l));
  return o;
}
__device__ __forceinline__ BestEntry wave_best(BestEntry e) {
  best_offer_dpp<kDppQuadXor1>(e);
  best_offer_dpp<kDppQuadXor2>(e);
  best_offer_dpp<kDppRowHalfMirror>(e);
  best_offer_dpp<kDppRowMirror>(e);
  BestEntry a = best_readlane(e, 0), b = best_readlane(e, 16), c = best_readlane(e, 32), d = best_readlane(e, 48);
  best_offer(a, b.slot, b.s, b.m);
  best_offer(c, d.slot, d.s, d.m);
  best_offer(a, c.slot, c.s, c.m);
  return a;
}

// 64 candidates, one per lane: the W2 run [kb, kb + 8 KQ) of this lane's
// candidate row, as stored, with its id, base value and bias.  score() adds the
// wave's partial dot products over [kb, ke), taking bottleneck value kb + i
// from lane i of the wave (av; read as a uniform value, so no LDS is
// involved; runs past ke take zero weights through selects), and lets wave 0
// sum the waves' partials in wave order.
template <class W, int KQ>
struct ScoreBatch {
  uint4 w[KQ * sizeof(W) / 2];  // 8 bf16 per uint4, or 4 floats
  int v;
  float cv, bf;
  __device__ __forceinline__ void load(const TreeArgs& t, const int32_t* cidx, const float* cval, int j0, int M,
                                       int kb) {
    const int lane = threadIdx.x & 63, r = t.r;
    const int j = min(j0 + lane, M - 1);
    v = cidx[j];
    cv = cval[j];
    const W* row = reinterpret_cast<const W*>(t.w2) + (size_t)v * r;
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
      const W* p = row + min(kb + 8 * q, r - 8);
      if constexpr (sizeof(W) == 2) {
        w[q] = *reinterpret_cast<const uint4*>(p);
      } else {
        w[2 * q] = *reinterpret_cast<const uint4*>(p);
        w[2 * q + 1] = *reinterpret_cast<const uint4*>(p + 4);
      }
    }
    bf = t.b2 ? t.b2[v] : 0.f;
  }
  // this wave's partial dot product of the lane's candidate, into part[wv][lane]
  __device__ __forceinline__ void partial(double av, double (*part)[64], int kb, int ke) const {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    double sdot = 0.0;
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
      const bool in = kb + 8 * q < ke;
      double x[8];
      if constexpr (sizeof(W) == 2) {
        bf16x8_to_f64(w[q], x);
      } else {
        const uint4 u0 = w[2 * q], u1 = w[2 * q + 1];
        x[0] = __uint_as_float(u0.x), x[1] = __uint_as_float(u0.y), x[2] = __uint_as_float(u0.z);
        x[3] = __uint_as_float(u0.w), x[4] = __uint_as_float(u1.x), x[5] = __uint_as_float(u1.y);
        x[6] = __uint_as_float(u1.z), x[7] = __uint_as_float(u1.w);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sdot += (in ? x[e] : 0.0) * readlane_f64(av, 8 * q + e);
    }
    part[wv][lane] = sdot;
  }
  // after a barrier: the corrected logit of the lane's candidate (wave 0)
  template <int NWV>
  __device__ __forceinline__ double logit(const double (*part)[64]) const {
    const int lane = threadIdx.x & 63;
    double tot = part[0][lane];
#pragma unroll
    for (int u = 1; u < NWV; ++u) tot += part[u][lane];
    return (double)cv + (double)bf + tot;
  }
};

// Round k of sequence b: score the current node's M children, push them, pop
// the best entry; one workgroup of NWV waves.  Wave w scores candidates w,
// w + NWV, ...: lanes split the bottleneck in runs of 4 and the partial dot
// products are reduced across the wave.  kLL (one launch per round): the
// bottleneck arrives as round k's hand-off words, and the popped node also
// goes out as hand-off words (tag) for the GRU step of round k + 1 in the same
// launch; the first batch of candidate rows is read before the bottleneck.
template <class W, int NWV, bool kLL>
__device__ __forceinline__ void score_pop(const TreeArgs& t, int b, int k, uint32_t tag) {
  __shared__ double l[256];     // corrected candidate logits (M <= 256)
  __shared__ int lid[256];      // their token ids
  __shared__ double part[NWV][64];  // the waves' partial dot products of 64 candidates
  __shared__ double lse_s;
  __shared__ BestEntry wbest[NWV];
  __shared__ double last_s;     // the last entry pushed
  __shared__ int4 last_m;
  __shared__ int next_depth;    // depth of the node the next round expands, or -1
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = t.r, M = t.M, P = t.P;
  // the bottleneck does not depend on the cursor: its read goes out first.
  // Candidates go 64 at a time, one per lane; wave w takes the k range
  // [w kc, w kc + kc) of every candidate's W2 row (its reads go out before
  // the bottleneck is needed) and the waves' partial dot products meet in
  // LDS, added in wave order: no cross-lane reduction per candidate.  Lane i
  // of wave w holds bottleneck value w kc + i (mod the KW lanes a range can
  // span).
  constexpr int KQ = 256 / NWV / 8, KW = 8 * KQ;  // runs of 8 k values per lane and wave (r <= 256)
  const int kc = ((r + NWV - 1) / NWV + 7) & ~7;
  const int kb = min(wv * kc, r), ke = min(kb + kc, r);
  const int arow = min(kb + (lane & (KW - 1)), r - 1);
  double av = 0.0;
  if constexpr (!kLL) av = t.act[(size_t)b * r + arow];
  const TreeCur c = tree_cur(t, k)[b];
  double* hs = t.heap_score + (size_t)b * t.heap_cap;
  int4* hm = t.heap_meta + (size_t)b * t.heap_cap;
  int count = t.heap_count[b];
  // each thread's best among the entries already on the heap, read before the
  // scoring so that no read has to follow the pushes (the heap order is a strict
  // total order, so the scan order does not matter); thread 0 also keeps the
  // last entry, which refills the popped slot when nothing is pushed
  BestEntry best = best_empty();
  for (int i0 = tid; i0 < count; i0 += 4 * (int)blockDim.x) {  // four reads in flight per thread
    double sv[4];
    int4 mv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = min(i0 + q * (int)blockDim.x, count - 1);
      sv[q] = hs[i];
      mv[q] = hm[i];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + q * (int)blockDim.x;
      best_offer(best, i, sv[q], mv[q], i < count);
    }
  }
  double tail_s = 0.0;
  int4 tail_m = make_int4(0, 0, 0, 0);
  if (tid == 0 && count > 0) {
    tail_s = hs[count - 1];
    tail_m = hm[count - 1];
  }

  if (c.expand) {
    const int delta = c.depth;
    const int32_t* cidx = t.cand_idx + ((size_t)b * P + delta) * M;
    const float* cval = t.cand_val + ((size_t)b * P + delta) * M;
    ScoreBatch<W, KQ> bt;
    bt.load(t, cidx, cval, 0, M, kb);
    if constexpr (kLL) {
      // the bottleneck of round k, one fp64 value (two words) per thread
      const uint64_t* src = t.ll_act + (((size_t)k * t.B + b) * r + arow) * 2;
      uint64_t w0 = 0, w1 = 0;
      ll_wait(t.status, [&] {
        w0 = ld_agent64(src);
        w1 = ld_agent64(src + 1);
        return (int)ll_ok(w0, tag) & (int)ll_ok(w1, tag);
      });
      av = __longlong_as_double((long long)(((uint64_t)ll_data(w1) << 32) | ll_data(w0)));
    }
    bt.partial(av, part, kb, ke);
    __syncthreads();
    if (M <= 64) {
      // one group: wave 0 finishes in registers (log-sum-exp over the M
      // candidates, the children's scores, their push) while the other waves
      // go on to the pop with their heap entries
      if (wv == 0) {
        const bool valid = lane < M;
        const double lj = bt.template logit<NWV>(part);
        const double mx = wave_max(valid ? lj : -INFINITY);
        const double se = wave_sum(valid ? exp(lj - mx) : 0.0);
        const double sj = c.score + (lj - (mx + log(se)));
        const int4 mj = make_int4(c.node, lane, bt.v, delta + 1);
        if (valid) {
          hs[count + lane] = sj;
          hm[count + lane] = mj;
          best_offer(best, count + lane, sj, mj);
        }
        if (lane == M - 1) {
          last_s = sj;
          last_m = mj;
        }
      }
    } else {
      for (int j0 = 0;;) {
        if (wv == 0 && j0 + lane < M) {
          l[j0 + lane] = bt.template logit<NWV>(part);
          lid[j0 + lane] = bt.v;
        }
        __syncthreads();  // part is reused by the next group
        j0 += 64;
        if (j0 >= M) break;
        bt.load(t, cidx, cval, j0, M, kb);
        bt.partial(av, part, kb, ke);
        __syncthreads();
      }
      // log-sum-exp over the M candidates (one wave)
      if (wv == 0) {
        double mx = -INFINITY;
        for (int j = lane; j < M; j += 64) mx = fmax(mx, l[j]);
        mx = wave_max(mx);
        double se = 0.0;
        for (int j = lane; j < M; j += 64) se += exp(l[j] - mx);
        se = wave_sum(se);
        if (lane == 0) lse_s = mx + log(se);
      }
      __syncthreads();
      const double lse = lse_s;
      for (int j = tid; j < M; j += blockDim.x) {
        const double sj = c.score + (l[j] - lse);
        const int4 mj = make_int4(c.node, j, lid[j], delta + 1);
        hs[count + j] = sj;
        hm[count + j] = mj;
        best_offer(best, count + j, sj, mj);
        if (j == M - 1) {
          last_s = sj;
          last_m = mj;
        }
      }
    }
    count += M;
  }

  // pop: best entry under (score desc, parent asc, rank asc): within each
  // wave by shuffles, then over the waves
  best = wave_best(best);
  if (lane == 0) wbest[wv] = best;
  __syncthreads();
  if (tid == 0) {
    BestEntry e = wbest[0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) best_offer(e, wbest[w].slot, wbest[w].s, wbest[w].m);
    const size_t o = (size_t)b * t.N + k;
    const int bi = e.slot;
    const double s = e.s;
    const int4 m = e.m;
    TreeCur n;
    n.slot = k + 1;
    n.node = k;
    n.expand = bi >= 0 && m.w < P && k + 1 < t.N ? 1 : 0;
    n.parent_slot = bi >= 0 ? m.x + 1 : -1;  // node index -> state slot; the anchor's slot is 0
    n.token = bi >= 0 ? m.z : 0;
    n.depth = bi >= 0 ? m.w : 0;
    n.score = bi >= 0 ? s : 0.0;
    // the next round's GRU step waits for the popped node: it goes out first
    if constexpr (kLL) {
      if (k + 1 < t.N) {
        uint64_t* w = t.ll_cur + ((size_t)k * t.B + b) * 2;
        ll_put(w, (uint32_t)n.token, tag);
        ll_put(w + 1, (uint32_t)(n.parent_slot + 1) | ((uint32_t)n.expand << 16), tag);
      }
    }
    if (bi < 0) {
      t.out_parents[o] = -1;
      t.out_tokens[o] = -1;
      if (t.out_depth) t.out_depth[o] = 0;
      if (t.out_scores) t.out_scores[o] = -INFINITY;
    } else {
      t.out_parents[o] = m.x;
      t.out_tokens[o] = m.z;
      if (t.out_depth) t.out_depth[o] = m.w;
      if (t.out_scores) t.out_scores[o] = s;
      // the last entry moves into the popped slot
      if (c.expand) {
        hs[bi] = last_s;
        hm[bi] = last_m;
      } else {
        hs[bi] = tail_s;
        hm[bi] = tail_m;
      }
      count -= 1;
    }
    t.heap_count[b] = count;
    tree_cur(t, k + 1)[b] = n;
    next_depth = n.expand ? n.depth : -1;
  }
  // the H half at the depth of the node the next round expands, for its bottleneck
  __syncthreads();
  const int nd = next_depth;
  if (nd >= 0)
    for (int i = tid; i < r; i += blockDim.x) t.zh_cur[(size_t)b * r + i] = t.zh[((size_t)b * P + nd) * r + i];
}

template <class W>
__global__ __launch_bounds__(256) void tree_score_pop(TreeArgs t, int k) {
  score_pop<W, 4, false>(t, blockIdx.x, k, 0u);
}

// After the top-M segments, in one launch: each row's merge of its segment
// lists, the H half of the bottleneck in fp64 (tree_zh tiles), the per-call
// set-up and, with bf16 weights, round 0's GRU step (the anchor, whose token
// is a first token and whose parent state is zero), on workgroups of 8 waves;
// none reads what another writes.
template <class W, bool kTab>
__global__ __launch_bounds__(64 * kZhWaves) void tree_prep(TreeArgs t) {
  static_assert(kZhWaves == kGruWaves, "one workgroup size for every part");
  const int rows = t.B * t.P, nzk = (t.r + 15) / 16, nzm = (rows + 15) / 16, wg = blockIdx.x;
  const int nz = rows + nzk * nzm;
  if (wg < rows) {
    merge_row(t.seg_keys, t.M, t.cand_idx, t.cand_val, wg);
  } else if (wg < nz) {
    const int z = wg - rows;
    zh_tile<W>(t, z % nzk, z / nzk);
  } else if (wg == nz) {
    tree_init(t);
  } else if constexpr (sizeof(W) == 2) {
    const int g = wg - nz - 1, nu = (t.Hs + 3) / 4;
    gru_mfma_step<kTab, false>(t, (g / nu) * kTreeSeqs, g - (g / nu) * nu, 0, 0u);
  }
}

// ---- one launch per round (bf16 weights) ------------------------------------------------------
// Launch k runs round k's bottleneck, its score and pop, and the GRU step of
// round k + 1, in workgroups of 8 waves numbered in that order: ceil(r / 32)
// per sequence for the bottleneck (four rows per wave), one per sequence for
// the score and pop, ceil(Hs / 4) per group of kTreeSeqs sequences for the
// GRU.  The bottleneck and the popped node pass between them as tagged
// hand-off words; everything else a round reads was written by an earlier
// launch.  A workgroup waits only for lower-numbered ones (score on
// bottleneck, GRU on score), and each XCD starts its workgroups in order, so
// the waits end whether or not all workgroups fit on the device at once.
template <bool kTab>
__global__ __launch_bounds__(64 * kGruWaves) void tree_round(TreeArgs t, int k) {
  const uint32_t tag = ll_tag(*t.epoch, k);
  const int nr = (t.r + 31) / 32, nbt = nr * t.B, wg = blockIdx.x;
  if (wg < nbt) {
    const int b = wg / nr;
    bottleneck_rows<uint16_t, true>(t, b, (wg - b * nr) * 32 + (threadIdx.x >> 6) * 4, k, tag);
  } else if (wg < nbt + t.B) {
    score_pop<uint16_t, kGruWaves, true>(t, wg - nbt, k, tag);
  } else {
    const int g = wg - nbt - t.B, nu = (t.Hs + 3) / 4;
    if constexpr (kTab)
      gru_tab_ll_step(t, (g / nu) * kTreeSeqs, g - (g / nu) * nu, k + 1, tag);
    else
      gru_mfma_step<false, true>(t, (g / nu) * kTreeSeqs, g - (g / nu) * nu, k + 1, tag);
  }
}

// ---- host side ------------------------------------------------------------------------------
static size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

size_t topm_scratch_bytes(int rows, int M) { return al256((size_t)rows * kTopSegs * M * 8); }

TreeLayout tree_layout(int d, int Hs, int r, int P, int group, int N, int M) {
  (void)d;
  TreeLayout L;
  size_t off = 0;
  L.status = off;
  off += 256;
  L.seg_keys = off;
  off += topm_scratch_bytes(group * P, M);
  L.cand_idx = off;
  off += al256((size_t)group * P * M * 4);
  L.cand_val = off;
  off += al256((size_t)group * P * M * 4);
  L.zh = off;
  off += al256((size_t)group * P * r * 8);
  L.zh_cur = off;
  off += al256((size_t)group * r * 8);
  L.act = off;
  off += al256((size_t)group * r * 8);
  L.states = off;
  off += al256((size_t)group * (N + 1) * Hs * 8);
  L.gh = off;
  off += al256((size_t)group * (N + 1) * 3 * Hs * 8);
  L.heap_cap = N * M;
  L.heap_score = off;
  off += al256((size_t)group * L.heap_cap * 8);
  L.heap_meta = off;
  off += al256((size_t)group * L.heap_cap * 16);
  L.heap_count = off;
  off += al256((size_t)group * 4);
  L.cur = off;
  off += al256((size_t)2 * group * sizeof(TreeCur));  // two slots (round parity)
  L.ll_act = off;
  off += al256((size_t)N * group * r * 16);
  L.ll_cur = off;
  off += al256((size_t)N * group * 16);
  L.total = off;
  return L;
}

static hipError_t launch_topm_impl(const float* Lb, int rows, int V, int M, uint64_t* seg, int32_t* idx, float* val,
                                   int32_t* status, bool reset_status, hipStream_t s) {
  hipLaunchKernelGGL(topm_segment, dim3(kTopSegs, rows), dim3(256), 0, s, Lb, V, M, seg, status, reset_status ? 1 : 0);
  hipLaunchKernelGGL(topm_merge, dim3(rows), dim3(256), 0, s, seg, M, idx, val);
  return hipGetLastError();
}

hipError_t launch_topm(const float* Lb, int rows, int V, int M, void* scratch, int32_t* idx, float* val, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return launch_topm_impl(Lb, rows, V, M, (uint64_t*)scratch, idx, val, nullptr, false, s);
}

// LDS of the GRU-step kernel that runs for this storage type, static part included
size_t tree_gru_lds_total(int d, int Hs, int dtype) {
  if (dtype == kBF16) return sizeof(double) * kGruWaves * 2 * 12 * kTreeSeqs;  // static only, any shape
  return tree_gru_lds(d, Hs, dtype) + sizeof(TreeCur) * kTreeSeqs;
}

size_t tree_gru_lds(int d, int Hs, int dtype) {
  return (size_t)kTreeSeqs * Hs * sizeof(double) + (size_t)kTreeSeqs * d * (dtype == kBF16 ? 2 : 4);
}

hipError_t launch_tree(const TreeArgs& t, bool reset_status, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (t.B <= 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (ev_start && ev_stop && (e = hipEventRecord(ev_start, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(topm_segment, dim3(kTopSegs, t.B * t.P), dim3(256), 0, s, t.Lb, t.V, t.M, t.seg_keys, t.status,
                     reset_status ? 1 : 0);
  const int prep = t.B * t.P + (t.r + 15) / 16 * ((t.B * t.P + 15) / 16) + 1;
  const int ngr0 = (t.Hs + 3) / 4 * ((t.B + kTreeSeqs - 1) / kTreeSeqs);  // round 0's GRU workgroups (bf16)
  if (t.dtype == kBF16 && t.xt)
    hipLaunchKernelGGL((tree_prep<uint16_t, true>), dim3(prep + ngr0), dim3(64 * kZhWaves), 0, s, t);
  else if (t.dtype == kBF16)
    hipLaunchKernelGGL((tree_prep<uint16_t, false>), dim3(prep + ngr0), dim3(64 * kZhWaves), 0, s, t);
  else
    hipLaunchKernelGGL((tree_prep<float, false>), dim3(prep), dim3(64 * kZhWaves), 0, s, t);
  // bf16 weights: the GRU step on the fp64 matrix cores (static LDS only)
  const bool mfma = t.dtype == kBF16;
  const size_t lds = mfma ? 0 : tree_gru_lds(t.d, t.Hs, t.dtype);
  static thread_local size_t attr_lds = 0;
  if (!mfma && lds > attr_lds) {
    e = hipFuncSetAttribute((const void*)tree_gru, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_lds = lds;
  }
  if (mfma) {
    // bf16 weights (round 0's GRU step ran in tree_prep): one launch per round
    // (round k's bottleneck, score and pop, and round k + 1's GRU step)
    const int nbt = (t.r + 31) / 32 * t.B, ngr = (t.Hs + 3) / 4 * ((t.B + kTreeSeqs - 1) / kTreeSeqs);
    for (int k = 0; k < t.N; ++k) {
      const int grid = nbt + t.B + (k + 1 < t.N ? ngr : 0);
      if (t.xt)
        hipLaunchKernelGGL(tree_round<true>, dim3(grid), dim3(64 * kGruWaves), 0, s, t, k);
      else
        hipLaunchKernelGGL(tree_round<false>, dim3(grid), dim3(64 * kGruWaves), 0, s, t, k);
    }
  } else {
    for (int k = 0; k < t.N; ++k) {
      for (int b0 = 0; b0 < t.B; b0 += kTreeSeqs)
        hipLaunchKernelGGL(tree_gru, dim3((t.Hs + 3) / 4), dim3(64 * 4 * (kTreeSeqs / kSeqPerWave)), lds, s, t, b0, k);
      hipLaunchKernelGGL(tree_bottleneck<float>, dim3((t.r + 15) / 16, t.B), dim3(256), 0, s, t, k);
      hipLaunchKernelGGL(tree_score_pop<float>, dim3(t.B), dim3(256), 0, s, t, k);
    }
  }
  e = hipGetLastError();
  if (e == hipSuccess && ev_start && ev_stop) e = hipEventRecord(ev_stop, s);
  return e;
}

}  // namespace dh
