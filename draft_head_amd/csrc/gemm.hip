// "NT" matrix products on the MFMA matrix cores:
//   C[m][n] = sum_k A[m][k] * B[n][k]      (fp32 accumulate, fp32 out)
// A is the activation side (rows = draft-block positions), B the weight side
// (rows = vocabulary entries or bottleneck units); both are k-contiguous.
// Used for the block-parallel base logits Lb = H W_lm^T through the frozen LM
// head (Dutch Domino summary, "Methodologie", part 1; 163.com explainer,
// section 3) and for the H-half of the bottleneck projection, W1[:, :d] H_i.
//
// Two kernels:
//  * gemm_stream: every wave owns 16 columns (16 weight rows) and streams
//    their full k range from HBM straight into MFMA fragments; each
//    workgroup row covers MT 16-row tiles of A.  For few activation rows
//    the product is bound by reading B once, so nothing is staged in LDS.
//  * gemm_tiled: 128x128 output tiles, k staged through LDS in 64-deep
//    slabs (double buffered), 2x2 waves of 64x64, bf16 only.  Tiles that
//    share B columns are issued to the same XCD so they meet in its L2.
#include "device.h"
#include "internal.h"

namespace dh {

#ifndef DH_STREAM_NT
#define DH_STREAM_NT 2  // 16-column tiles per wave
#endif
#ifndef DH_STREAM_U
#define DH_STREAM_U 4   // k chunks per batch of loads
#endif

// Each wave owns NT adjacent 16-column tiles and MT 16-row tiles of A, so one
// A fragment feeds NT MFMAs and one B fragment MT MFMAs.
template <class W, int MT, int NT>
__global__ __launch_bounds__(256) void gemm_stream(const W* __restrict__ A, int lda, const W* __restrict__ B, int ldb,
                                                   float* __restrict__ C, int ldc, int M, int N, int K) {
  constexpr int U = sizeof(W) == 2 ? DH_STREAM_U : (DH_STREAM_U > 2 ? DH_STREAM_U / 2 : 1);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * 4 + wv) * 16 * NT;
  if (n0 >= N) return;
  const int row = lane & 15, kg = lane >> 4;
  const int m_base = blockIdx.y * MT * 16;
  // rows past the end read a valid row; their results are never stored
  const W* brow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) brow[j] = B + (size_t)min(n0 + j * 16 + row, N - 1) * ldb + kg * 8;
  const W* arow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) arow[t] = A + (size_t)min(m_base + t * 16 + row, M - 1) * lda + kg * 8;

  f32x4 acc[MT][NT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nck = (K + 31) / 32;
  for (int c0 = 0; c0 < nck; c0 += U) {
    frag_t<W> bf[U][NT];
    frag_t<W> af[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (c0 + u) * 32;
      const bool ok = k + kg * 8 < K;
#pragma unroll
      for (int j = 0; j < NT; ++j) bf[u][j] = load8_or_zero(brow[j] + k, ok);
#pragma unroll
      for (int t = 0; t < MT; ++t) af[u][t] = load8_or_zero(arow[t] + k, ok);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[t][j] = mma(af[u][t], bf[u][j], acc[t][j]);
  }

#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int n = n0 + j * 16 + row;
    if (n >= N) continue;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m_base + t * 16 + kg * 4 + i;
        if (m < M) C[(size_t)m * ldc + n] = acc[t][j][i];
      }
  }
}

#ifndef DH_R16_WAVES
#define DH_R16_WAVES 8  // waves per workgroup of gemm_rows16
#endif
#ifndef DH_R16_U
#define DH_R16_U 8      // k chunks per batch of loads in gemm_rows16
#endif

// At most 16 rows of A (one draft block of one sequence): the product is
// bound by reading B once, and what limits the rate is how evenly that read
// is spread.  Persistent: one workgroup per CU; A is staged once in LDS in
// fragment order (k chunk c, lane l at 16-byte slot c*64 + l, so a fragment
// read is 1 KB contiguous).  Workgroup g owns the 16-column tiles
// [T g / G, T (g+1) / G); its waves split that range's (tile, k chunk) pairs
// evenly, so every wave streams the same number of bytes of B.  A tile cut
// between waves w and w+1 is finished by wave w as its lower-k part plus
// wave w+1's higher-k part, a fixed order.  Needs at least WAVES tiles per
// workgroup, so no tile is cut twice.
template <int WAVES, int U>
__global__ __launch_bounds__(64 * WAVES) void gemm_rows16(const uint16_t* __restrict__ A, int lda,
                                                          const uint16_t* __restrict__ B, int ldb, float* __restrict__ C,
                                                          int ldc, int M, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) uint4 sA[];  // [k chunks][64 lanes]
  __shared__ __attribute__((aligned(16))) float4 part[WAVES][64];
  const int nck = (K + 31) / 32;
  for (int q = threadIdx.x; q < nck * 64; q += blockDim.x) {
    const int c = q >> 6, l = q & 63, r = l & 15, k = c * 32 + (l >> 4) * 8;
    sA[q] = (r < M && k < K) ? *reinterpret_cast<const uint4*>(A + (size_t)r * lda + k) : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15, kg = lane >> 4;
  const int T = (N + 15) / 16, G = gridDim.x, g = blockIdx.x;
  const int tb = (int)((int64_t)T * g / G), te = (int)((int64_t)T * (g + 1) / G);
  const int64_t total = (int64_t)(te - tb) * nck;
  const int64_t lo = total * wv / WAVES, hi = total * (wv + 1) / WAVES;

  auto store_tile = [&](int t, const f32x4& v) {
    const int n = t * 16 + row;
    if (n >= N) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (kg * 4 + i < M) C[(size_t)(kg * 4 + i) * ldc + n] = v[i];
  };

  f32x4 head = {0.f, 0.f, 0.f, 0.f};  // lower-k part of the tile cut at the end of this wave's range
  int cut_tile = -1;
  for (int64_t pos = lo; pos < hi;) {
    const int t = tb + (int)(pos / nck), c0 = (int)(pos % nck);
    const int c1 = (int)(c0 + (hi - pos) < nck ? c0 + (hi - pos) : nck);
    const uint16_t* brow = B + (size_t)min(t * 16 + row, N - 1) * ldb + kg * 8;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c = c0; c < c1; c += U) {
      bf16x8 bfr[U], af[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int cc = c + u;
        const bool ok = cc < c1 && cc * 32 + kg * 8 < K;
        bfr[u] = load8_or_zero(brow + cc * 32, ok);
        af[u] = ok ? __builtin_bit_cast(bf16x8, sA[cc * 64 + lane]) : zero8<uint16_t>();
      }
#pragma unroll
      for (int u = 0; u < U; ++u) acc = mma(af[u], bfr[u], acc);
    }
    if (c0 == 0 && c1 == nck) {
      store_tile(t, acc);
    } else if (c0 == 0) {  // the range ends inside tile t
      head = acc;
      cut_tile = t;
    } else {  // the range starts inside tile t: its higher-k part
      part[wv][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    pos += c1 - c0;
  }
  __syncthreads();
  if (cut_tile >= 0) {
    const float4 q = part[wv + 1][lane];
    store_tile(cut_tile, f32x4{head[0] + q.x, head[1] + q.y, head[2] + q.z, head[3] + q.w});
  }
}

// Small products (few columns, e.g. the 256 bottleneck units): one 16x16
// output tile per workgroup, k split over its 4 waves (splitk_tile).
template <class W>
__global__ __launch_bounds__(256) void gemm_splitk(const W* __restrict__ A, int lda, const W* __restrict__ B, int ldb,
                                                   float* __restrict__ C, int ldc, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) float red[4 * 64 * 4];
  splitk_tile<W>(A, lda, B, ldb, C, ldc, M, N, K, blockIdx.x, blockIdx.y, red);
}

constexpr int TBM = 128, TBN = 128, TBK = 64, TPAD = 8;

__global__ __launch_bounds__(256) void gemm_tiled(const uint16_t* __restrict__ A, int lda,
                                                  const uint16_t* __restrict__ B, int ldb, float* __restrict__ C,
                                                  int ldc, int M, int N, int K, int m_tiles, int n_tiles,
                                                  int per_xcd) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][TBM][TBK + TPAD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][TBN][TBK + TPAD];

  // blocks are dealt to the 8 XCDs round-robin; give each XCD a contiguous
  // run of tiles, m fastest, so the m tiles of one n tile share an L2
  const int bid = blockIdx.x;
  const int t = (bid & 7) * per_xcd + (bid >> 3);
  if (t >= m_tiles * n_tiles) return;
  const int mt = t % m_tiles, nt = t / m_tiles;
  const int m0 = mt * TBM, n0 = nt * TBN;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int row = lane & 15, kg = lane >> 4;

  // global -> LDS assignment: 1024 16-byte pieces per operand tile, 4 per thread
  int g_row[4], g_col[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i;
    g_row[i] = q >> 3;
    g_col[i] = (q & 7) * 8;
  }
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a_src[i] = A + (size_t)min(m0 + g_row[i], M - 1) * lda + g_col[i];
    b_src[i] = B + (size_t)min(n0 + g_row[i], N - 1) * ldb + g_col[i];
  }

  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = k0 + g_col[i] < K;
      ra[i] = ok ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
      rb[i] = ok ? *reinterpret_cast<const uint4*>(b_src[i] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(&sA[buf][g_row[i]][g_col[i]]) = ra[i];
      *reinterpret_cast<uint4*>(&sB[buf][g_row[i]][g_col[i]]) = rb[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + TBK - 1) / TBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) gload((ks + 1) * TBK);
#pragma unroll
    for (int kc = 0; kc < TBK / 32; ++kc) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = load8(&sA[buf][wm * 64 + i * 16 + row][kc * 32 + kg * 8]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = load8(&sB[buf][wn * 64 + j * 16 + row][kc * 32 + kg * 8]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma(af[i], bfr[j], acc[i][j]);
    }
    if (ks + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 64 + j * 16 + row;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * 64 + i * 16 + kg * 4 + e;
        if (m < M) C[(size_t)m * ldc + n] = acc[i][j][e];
      }
  }
}

template <class W>
static hipError_t launch_stream(const W* A, int lda, const W* B, int ldb, float* C, int ldc, int M, int N, int K,
                                hipStream_t s) {
  constexpr int NT = DH_STREAM_NT;
  const int n_waves = (N + 16 * NT - 1) / (16 * NT);
  const int m_tiles = (M + 15) / 16;
  const int mt = m_tiles >= 4 ? 4 : (m_tiles >= 2 ? 2 : 1);
  dim3 grid((n_waves + 3) / 4, (m_tiles + mt - 1) / mt);
  if (mt == 4)
    hipLaunchKernelGGL((gemm_stream<W, 4, NT>), grid, dim3(256), 0, s, A, lda, B, ldb, C, ldc, M, N, K);
  else if (mt == 2)
    hipLaunchKernelGGL((gemm_stream<W, 2, NT>), grid, dim3(256), 0, s, A, lda, B, ldb, C, ldc, M, N, K);
  else
    hipLaunchKernelGGL((gemm_stream<W, 1, NT>), grid, dim3(256), 0, s, A, lda, B, ldb, C, ldc, M, N, K);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(int dtype, const void* A, int lda, const void* B, int ldb, float* C, int ldc, int M, int N,
                          int K, bool prefer_tiles, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (N <= 4096) {  // few columns: split k inside each workgroup
    dim3 grid((N + 15) / 16, (M + 15) / 16);
    if (dtype == kF32)
      hipLaunchKernelGGL(gemm_splitk<float>, grid, dim3(256), 0, s, (const float*)A, lda, (const float*)B, ldb, C, ldc,
                         M, N, K);
    else
      hipLaunchKernelGGL(gemm_splitk<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)A, lda, (const uint16_t*)B,
                         ldb, C, ldc, M, N, K);
    return hipGetLastError();
  }
  if (dtype == kF32)
    return launch_stream((const float*)A, lda, (const float*)B, ldb, C, ldc, M, N, K, s);
  if (M <= 16) {
    constexpr int WV = DH_R16_WAVES;
    const int cus = device_cus();
    const size_t lds = (size_t)((K + 31) / 32) * 64 * 16;
    if (cus > 0 && (N + 15) / 16 >= WV * cus && lds <= 128 * 1024) {
      static thread_local int attr_device = -1;
      int dev = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e != hipSuccess) return e;
      if (attr_device != dev) {
        e = hipFuncSetAttribute((const void*)gemm_rows16<WV, DH_R16_U>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                128 * 1024);
        if (e != hipSuccess) return e;
        attr_device = dev;
      }
      hipLaunchKernelGGL((gemm_rows16<WV, DH_R16_U>), dim3(cus), dim3(64 * WV), lds, s, (const uint16_t*)A, lda,
                         (const uint16_t*)B, ldb, C, ldc, M, N, K);
      return hipGetLastError();
    }
  }
  if (!prefer_tiles || M <= 64)
    return launch_stream((const uint16_t*)A, lda, (const uint16_t*)B, ldb, C, ldc, M, N, K, s);
  const int m_tiles = (M + TBM - 1) / TBM, n_tiles = (N + TBN - 1) / TBN;
  const int total = m_tiles * n_tiles;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL(gemm_tiled, dim3(per_xcd * 8), dim3(256), 0, s, (const uint16_t*)A, lda, (const uint16_t*)B,
                     ldb, C, ldc, M, N, K, m_tiles, n_tiles, per_xcd);
  return hipGetLastError();
}

}  // namespace dh
