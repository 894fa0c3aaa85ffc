// Device-side building blocks shared by the gfx950 kernels of this library.
//
// Fragment convention (one 64-lane wavefront, MFMA 16x16 with a 32-deep k chunk):
//   lane l supplies row (l % 16) of the left operand and column (l % 16) of
//   the right operand, each as 8 consecutive k values starting at
//   k0 + 8 * (l / 16).  Both operands use the same lane -> k map, so the
//   instruction's internal k order does not matter.  The 16x16 fp32 result
//   lands as: lane l holds column (l % 16), rows 4 * (l / 16) + 0..3.
//
// Storage types: bf16 (uint16_t bit patterns) or fp32.  bf16 x bf16
// products are exact in fp32; fp32 activations (GRU state, bottleneck)
// meet bf16 weights as a hi + lo pair of bf16 values (two MFMAs), which
// keeps about 16 significant bits of the activation instead of 8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dh {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct f32x8 {
  float4 lo, hi;
};

struct bf16pair {
  bf16x8 hi, lo;
};

// ---- scalar conversions ---------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even; inputs are finite
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- fragment loads -----------------------------------------------------------
__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ f32x8 load8(const float* p) {
  f32x8 r;
  r.lo = reinterpret_cast<const float4*>(p)[0];
  r.hi = reinterpret_cast<const float4*>(p)[1];
  return r;
}
template <class W>
struct frag;
template <>
struct frag<uint16_t> {
  using type = bf16x8;
};
template <>
struct frag<float> {
  using type = f32x8;
};
template <class W>
using frag_t = typename frag<W>::type;

template <class W>
__device__ __forceinline__ frag_t<W> zero8();
template <>
__device__ __forceinline__ bf16x8 zero8<uint16_t>() {
  return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
}
template <>
__device__ __forceinline__ f32x8 zero8<float>() {
  f32x8 r;
  r.lo = make_float4(0.f, 0.f, 0.f, 0.f);
  r.hi = r.lo;
  return r;
}

// 8 consecutive elements, or zeros when `ok` is false (no memory access then)
template <class W>
__device__ __forceinline__ frag_t<W> load8_or_zero(const W* p, bool ok) {
  return ok ? load8(p) : zero8<W>();
}

// ---- fp32 activations as right-hand operands ---------------------------------
__device__ __forceinline__ uint32_t pack2(uint16_t a, uint16_t b) { return (uint32_t)a | ((uint32_t)b << 16); }

__device__ __forceinline__ bf16pair split_hi_lo(const float4& x0, const float4& x1) {
  const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  uint16_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = f2bf(v[i]);
    l[i] = f2bf(v[i] - bf2f(h[i]));  // exact difference, then rounded
  }
  bf16pair r;
  r.hi = __builtin_bit_cast(bf16x8, make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])));
  r.lo = __builtin_bit_cast(bf16x8, make_uint4(pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])));
  return r;
}

// activation fragment type matching weight storage W
template <class W>
struct act;
template <>
struct act<uint16_t> {
  using type = bf16pair;
  __device__ static __forceinline__ type zero() {
    bf16pair r;
    r.hi = zero8<uint16_t>();
    r.lo = r.hi;
    return r;
  }
  __device__ static __forceinline__ type from_f32(const float* p) {
    const float4* q = reinterpret_cast<const float4*>(p);
    return split_hi_lo(q[0], q[1]);
  }
};
template <>
struct act<float> {
  using type = f32x8;
  __device__ static __forceinline__ type zero() { return zero8<float>(); }
  __device__ static __forceinline__ type from_f32(const float* p) { return load8(p); }
};

template <class W>
__device__ __forceinline__ typename act<W>::type act_or_zero(const float* p, bool ok) {
  return ok ? act<W>::from_f32(p) : act<W>::zero();
}

// ---- MFMA on one 32-deep k chunk ------------------------------------------------
__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16pair& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b.lo, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b.hi, c, 0, 0, 0);
}
// fp32: eight 16x16x4 instructions; instruction i takes element i of every lane's 8
__device__ __forceinline__ f32x4 mma(const f32x8& a, const f32x8& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, c, 0, 0, 0);
}

// ---- one 16x16 tile of C = A B^T with k split over the waves ---------------------
// For narrow products: each wave sums its share of the k chunks, the partials
// meet in LDS and wave 0 writes the tile.
// One 16x16 output tile of C = A B^T over the k chunks of 32 in [c_begin,
// c_end) (all of k by default), split over the NWV waves of the workgroup:
// wave w takes chunks from c_begin + w * U on, U at a time, NWV * U apart; the
// waves' partial tiles (red: NWV x 64 float4) are added in wave order.
template <class W, int NWV, int U>
__device__ void splitk_tile_n(const W* __restrict__ A, int lda, const W* __restrict__ B, int ldb, float* __restrict__ C,
                              int ldc, int M, int N, int K, int n_tile, int m_tile, float* red, int c_begin = 0,
                              int c_end = -1) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int n0 = n_tile * 16, m0 = m_tile * 16;
  const W* brow = B + (size_t)min(n0 + row, N - 1) * ldb + kg * 8;
  const W* arow = A + (size_t)min(m0 + row, M - 1) * lda + kg * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nck = c_end < 0 ? (K + 31) / 32 : c_end;
  for (int c0 = c_begin + wv * U; c0 < nck; c0 += NWV * U) {
    frag_t<W> af[U], bf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (c0 + u) * 32;
      const bool ok = c0 + u < nck && k + kg * 8 < K;
      af[u] = load8_or_zero(arow + k, ok);
      bf[u] = load8_or_zero(brow + k, ok);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc = mma(af[u], bf[u], acc);
  }
  *reinterpret_cast<float4*>(&red[(wv * 64 + lane) * 4]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  if (wv == 0) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float4 q = *reinterpret_cast<const float4*>(&red[(w * 64 + lane) * 4]);
      v[0] += q.x;
      v[1] += q.y;
      v[2] += q.z;
      v[3] += q.w;
    }
    const int n = n0 + row;
    if (n < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + kg * 4 + i;
        if (m < M) C[(size_t)m * ldc + n] = v[i];
      }
    }
  }
  __syncthreads();
}

// the same with four waves, 8 chunks per batch (bf16) or 4 (fp32)
template <class W>
__device__ void splitk_tile(const W* __restrict__ A, int lda, const W* __restrict__ B, int ldb, float* __restrict__ C,
                            int ldc, int M, int N, int K, int n_tile, int m_tile, float* red) {
  splitk_tile_n<W, 4, sizeof(W) == 2 ? 8 : 4>(A, lda, B, ldb, C, ldc, M, N, K, n_tile, m_tile, red);
}

// ---- greedy argmax as one 64-bit max ------------------------------------------
// key = (order-preserving bits of the value) << 32 | (0xFFFFFFFF - index):
// the largest key has the largest value and, among equal values, the lowest
// index.  -0.0 is folded to +0.0 first.  Key 0 is below every real key.
__device__ __forceinline__ uint64_t amax_key(float v, uint32_t idx) {
  if (v == 0.0f) v = 0.0f;
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ int32_t amax_index(uint64_t key) { return (int32_t)(0xFFFFFFFFu - (uint32_t)key); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// ---- bounded waits between workgroups of one persistent launch ------------------
// Every wait ends: on success, on a timeout already flagged by another wave,
// or after kWaitTicks of the 100 MHz constant clock (then it sets the status
// word to 2 itself).
constexpr uint64_t kWaitTicks = 200000000ull;  // 2 s
constexpr int kStatusTimeout = 2;  // same value as kDeviceStatusTimeout

// ---- tagged hand-off words ---------------------------------------------------------
// A value handed from one workgroup to others inside a persistent launch
// travels as one 64-bit word, 32 data bits under a 32-bit tag that names the
// launch and the step, written with a single agent-coherent 8-byte store
// (single-copy atomic) and read with agent-coherent loads.  Readers poll the
// words themselves until every tag is current: the data arrive with the
// signal, and a writer never waits for its stores to land.
__device__ __forceinline__ uint64_t ld_agent64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ll_put(uint64_t* w, uint32_t data, uint32_t tag) {
  __hip_atomic_store(w, ((uint64_t)tag << 32) | data, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool ll_ok(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }
// a workspace's hand-off words are cleared once (marker and layout signature
// written after); tags are epoch * 128 + step + 1 in 32 bits (steps < 64),
// with the epoch advanced once per call
constexpr uint64_t kLLMarker = 0x6c6c2d646f6d696eull;
constexpr uint32_t kEpochLimit = 1u << 25;
__host__ __device__ __forceinline__ uint32_t ll_tag(uint32_t epoch, int step) {
  return epoch * 128u + (uint32_t)step + 1u;
}
__device__ __forceinline__ uint32_t ll_data(uint64_t w) { return (uint32_t)w; }

// Repeat `attempt` (it issues the loads and tells, per lane, whether every
// word it read carries the expected tag) until it succeeds in every lane of
// the wave.  Gives up when another wave has flagged a timeout or after
// kWaitTicks (then flags one itself) and returns false; the caller carries on
// with what it read, so every wave still reaches the end of the kernel.  The
// shared flag and the clock are read on every 8th retry only: the flag read is
// a round trip to memory, and between two attempts it would double the time
// a wave takes to see words that have just landed.
// kSleep: s_sleep units (64 clocks each) between attempts; waits off the
// critical path use longer ones so they add less polling traffic.
template <int kSleep = 1, class F>
__device__ __forceinline__ bool ll_wait(int32_t* status, F&& attempt) {
  uint64_t t0 = 0;
  for (int tries = 0;; ++tries) {  // one call site, so `attempt` is inlined
    if (__all(attempt())) return true;
    if (tries == 0) {
      t0 = wall_clock64();
    } else if ((tries & 7) == 0) {
      if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == kStatusTimeout) return false;
      if (wall_clock64() - t0 > kWaitTicks) {
        __hip_atomic_store(status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(kSleep);
  }
}


// stores that are visible device-wide once complete (they bypass the
// per-XCD L2 write-back)
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dh
