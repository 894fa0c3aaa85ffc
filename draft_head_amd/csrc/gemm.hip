// "NT" matrix products on the MFMA matrix cores:
//   C[m][n] = sum_k A[m][k] * B[n][k]      (fp32 accumulate, fp32 out)
// A is the activation side (rows = draft-block positions), B the weight side
// (rows = vocabulary entries or bottleneck units); both are k-contiguous.
// Used for the block-parallel base logits Lb = H W_lm^T through the frozen LM
// head (Dutch Domino summary, "Methodologie", part 1; 163.com explainer,
// section 3) and for the H-half of the bottleneck projection, W1[:, :d] H_i.
//
// Kernels, by the number of rows of A:
//  * gemm_rows16 (at most 16 rows, one draft block): persistent, B streamed
//    once from HBM straight into MFMA fragments, A in LDS.
//  * gemm_stream (few rows, or fp32): every wave owns 16-column tiles and
//    streams their full k range; nothing is staged in LDS.
//  * gemm_tiled (up to 128 rows): 128x128 tiles, k staged through LDS.
//  * gemm_wide (more than 128 rows): persistent 256x256 tiles, direct
//    global->LDS loads; the product is then bound by how fast a CU can pull
//    operands from L2, so the tile is as large as the register file allows.
// Tiles that share B columns are given to the same XCD so they meet in its L2.
#include "device.h"
#include "internal.h"

namespace dh {

constexpr int kStreamNT = 2;  // 16-column tiles per wave of gemm_stream
constexpr int kStreamU = 4;   // k chunks per batch of loads

// Each wave owns NT adjacent 16-column tiles and MT 16-row tiles of A, so one
// A fragment feeds NT MFMAs and one B fragment MT MFMAs.
template <class W, int MT, int NT>
__global__ __launch_bounds__(256) void gemm_stream(const W* __restrict__ A, int lda, const W* __restrict__ B, int ldb,
                                                   float* __restrict__ C, int ldc, int M, int N, int K) {
  constexpr int U = sizeof(W) == 2 ? kStreamU : (kStreamU > 2 ? kStreamU / 2 : 1);
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

constexpr int kR16Waves = 16;  // waves per workgroup of gemm_rows16
constexpr int kR16U = 2;       // k chunks per batch of loads in gemm_rows16

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

// At most 16 rows of A, B read in whole-row pieces.  Streaming B in the MFMA
// fragment pattern (each load instruction: 16 rows x 64 B) reaches about 4.3
// TB/s on this part; 512-byte runs of single rows reach about 6 TB/s.  So each
// wave loads a "slab" of a 16-row tile, 256 k wide (two rows per instruction,
// eight instructions), two slabs ahead, writes the slab it is about to use to
// its own 8 KB of LDS and reads the B fragments back from there.  Row r's
// 16-byte unit u sits at unit position r * 32 + (u ^ r): both the writes and
// the fragment reads fall in distinct banks.  A is staged once in LDS in
// fragment order.  The workgroup's (tile, slab) pairs are split evenly over
// its waves; a tile cut between waves w and w + 1 is finished by wave w as
// its lower slabs plus wave w + 1's higher slabs, a fixed order.
//
// Output: scattered 64-byte stores issued while B streams cost about 13% of
// the kernel's time (stores share the load counter, and the partial-line
// writes land all over C's rows).  With STAGE, a wave keeps its finished
// tiles in registers (at most kR16Keep; the launch guarantees it), and at
// the end the workgroup assembles its whole column block in LDS and writes it
// row by row in 256-byte runs.  Loads use a wave-uniform base plus 32-bit lane
// offsets fixed for the whole kernel.
constexpr int kR16SlabK = 256;  // k per slab: 8 chunks of 32
constexpr int kR16Keep = 8;     // finished tiles a wave holds for the block store
template <int WAVES, bool STAGE>
__global__ __launch_bounds__(64 * WAVES) void gemm_rows16_slab(const uint16_t* __restrict__ A, int lda,
                                                               const uint16_t* __restrict__ B, int ldb,
                                                               float* __restrict__ C, int ldc, int M, int N, int K) {
  // [k chunks][64 lanes] of A, then WAVES slabs of 8 KB; after the main loop, the output block [16][cols]
  extern __shared__ __attribute__((aligned(16))) uint4 sA[];
  __shared__ __attribute__((aligned(16))) float4 part[WAVES][64];
  const int nck = K / 32, NS = K / kR16SlabK;
  for (int q = threadIdx.x; q < nck * 64; q += blockDim.x) {
    const int c = q >> 6, l = q & 63, r = l & 15, k = c * 32 + (l >> 4) * 8;
    sA[q] = r < M ? *reinterpret_cast<const uint4*>(A + (size_t)r * lda + k) : make_uint4(0, 0, 0, 0);
  }
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15, kg = lane >> 4, dr = lane >> 5, unit = lane & 31;
  unsigned char* slab = reinterpret_cast<unsigned char*>(sA + nck * 64) + (size_t)wv * 8192;
  const int T = (N + 15) / 16, G = gridDim.x, g = blockIdx.x;
  const int tb = (int)((int64_t)T * g / G), te = (int)((int64_t)T * (g + 1) / G);
  const int64_t total = (int64_t)(te - tb) * NS;
  const int64_t lo = total * wv / WAVES, hi = total * (wv + 1) / WAVES;
  const int t_lo = tb + (int)(lo / NS);
  const bool lo_cut = lo % NS != 0;  // the range starts inside tile t_lo
  uint32_t voff[8];                  // byte offsets of the lane's loads from a slab's start: row 2q + dr, unit
#pragma unroll
  for (int q = 0; q < 8; ++q) voff[q] = (uint32_t)((2 * q + dr) * ldb + unit * 8) * 2u;
  __syncthreads();

  // the loads of unit u (tile tb + u / NS, slab u % NS); past hi they repeat the last unit (never used)
  auto issue = [&](int64_t u, bf16x8 (&v)[8]) {
    const int64_t uu = u < hi ? u : hi - 1;
    const int t = tb + (int)(uu / NS), s = (int)(uu % NS);
    const unsigned char* base = reinterpret_cast<const unsigned char*>(B + (size_t)t * 16 * ldb + s * kR16SlabK);
    const int rmax = N - 1 - t * 16;
    if (rmax >= 15) {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = load8(reinterpret_cast<const uint16_t*>(base + voff[q]));
    } else {  // the last tile of a ragged B: rows past its end read its last row
#pragma unroll
      for (int q = 0; q < 8; ++q)
        v[q] = load8(reinterpret_cast<const uint16_t*>(base) + (size_t)min(2 * q + dr, rmax) * ldb + unit * 8);
    }
  };
  auto store_tile = [&](int t, const f32x4& v) {
    const int n = t * 16 + row;
    if (n >= N) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (kg * 4 + i < M) C[(size_t)(kg * 4 + i) * ldc + n] = v[i];
  };
  f32x4 kept[kR16Keep];
  int nkept = 0, tfirst = 0;  // kept[j] is tile tfirst + j: a wave's finished tiles are consecutive
  auto finish = [&](int t, const f32x4& v) {
    if (!STAGE) {
      store_tile(t, v);
      return;
    }
    if (nkept == 0) tfirst = t;
#pragma unroll
    for (int j = 0; j < kR16Keep; ++j)
      if (j == nkept) kept[j] = v;
    ++nkept;
  };
  f32x4 head = {0.f, 0.f, 0.f, 0.f};  // lower slabs of the tile cut at the end of this wave's range
  int cut_tile = -1;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  bf16x8 b0[8], b1[8], b2[8];
  if (lo < hi) {
    issue(lo, b0);
    issue(lo + 1, b1);
  }
  auto consume = [&](int64_t u, const bf16x8 (&v)[8]) {
    const int t = tb + (int)(u / NS), s = (int)(u % NS);
    if (s == 0 || u == lo) acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = 2 * q + dr;
      *reinterpret_cast<bf16x8*>(slab + (size_t)(r * 32 + (unit ^ r)) * 16) = v[q];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {  // the wave's own LDS writes above complete before these reads
      const bf16x8 bf = *reinterpret_cast<const bf16x8*>(slab + (size_t)(row * 32 + ((c * 4 + kg) ^ row)) * 16);
      const bf16x8 af = __builtin_bit_cast(bf16x8, sA[(s * 8 + c) * 64 + lane]);
      acc = mma(af, bf, acc);
    }
    const bool higher = t == t_lo && lo_cut;  // this wave holds only the higher slabs of tile t
    const bool last = s == NS - 1 || u == hi - 1;
    if (last) {
      if (higher) {
        part[wv][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      } else if (s == NS - 1) {
        finish(t, acc);
      } else {  // the range ends inside tile t
        head = acc;
        cut_tile = t;
      }
    }
  };
  int64_t u = lo;
  for (; u + 3 <= hi; u += 3) {
    issue(u + 2, b2);
    consume(u, b0);
    issue(u + 3, b0);
    consume(u + 1, b1);
    issue(u + 4, b1);
    consume(u + 2, b2);
  }
  if (u < hi) consume(u, b0);
  if (u + 1 < hi) consume(u + 1, b1);
  __syncthreads();  // part[] written; A and the slabs no longer read
  f32x4 joined = head;
  if (cut_tile >= 0) {
    const float4 q = part[wv + 1][lane];
    joined = f32x4{head[0] + q.x, head[1] + q.y, head[2] + q.z, head[3] + q.w};
    if (!STAGE) store_tile(cut_tile, joined);
  }
  if (STAGE) {
    float* blk = reinterpret_cast<float*>(sA);
    const int cols = (te - tb) * 16;
    auto put = [&](int t, const f32x4& v) {
#pragma unroll
      for (int i = 0; i < 4; ++i) blk[(kg * 4 + i) * cols + (t - tb) * 16 + row] = v[i];
    };
#pragma unroll
    for (int j = 0; j < kR16Keep; ++j)
      if (j < nkept) put(tfirst + j, kept[j]);
    if (cut_tile >= 0) put(cut_tile, joined);
    __syncthreads();
    const int c0 = tb * 16, cn = min(cols, N - c0);
    for (int q = threadIdx.x; q < M * cols; q += blockDim.x) {
      const int m = q / cols, c = q - m * cols;
      if (c < cn) C[(size_t)m * ldc + c0 + c] = blk[q];
    }
  }
}

constexpr int kWideBK = 64;   // k depth of a stage of gemm_wide
constexpr int kWideNBuf = 2;  // LDS stage buffers of gemm_wide

// Many rows of A, bf16, K a multiple of BK.
// Workgroup tile BM x BN (BM = 32 MT, BN = 64 NT), eight waves in 2 x 4, each
// MT x NT 16x16 tiles; k runs in BK-deep stages through a ring of NBUF LDS
// buffers.
// What bounds this product on MI355X is how fast a CU pulls operands from
// L2, so the tile is as large as the register file allows (fewer bytes per
// flop).  Loads go straight from global memory into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at slot l of a 1 KB
// block); a load covers 1024 / (2 BK) rows, lane l taking row l / (BK / 8)
// and 16-byte unit l % (BK / 8).  Row r's unit u is stored at position
// u ^ sw(r) of the row, sw chosen so that the 16 rows of a fragment read
// fall in distinct banks.  Persistent, one workgroup per CU, tiles dealt
// per XCD (below).  Stage q's loads are issued during stage
// q - (NBUF - 1) into the buffer that stage q - 1 used; the barrier at the
// end of every stage publishes the next one and frees the oldest.
template <int BK>
__device__ __forceinline__ int wide_swizzle(int r) {
  return BK == 64 ? (r >> 1) & 7 : (r >> 2) & 3;
}

template <int MT, int BK, int NBUF, int NT>
__global__ __launch_bounds__(512) void gemm_wide(const uint16_t* __restrict__ A, int lda,
                                                 const uint16_t* __restrict__ B, int ldb, float* __restrict__ C,
                                                 int ldc, int M, int N, int K, int m_tiles, int n_tiles) {
  static_assert(BK == 32 || BK == 64, "stage depth");
  constexpr int BM = 2 * MT * 16, BN = 4 * NT * 16;
  constexpr int ROWB = BK * 2, UPR = BK / 8, RPL = 64 / UPR;  // bytes, units per row; rows per load
  constexpr int A_BYTES = BM * ROWB, STAGE = A_BYTES + BN * ROWB;
  constexpr int A_LOADS = BM / RPL, LOADS = A_LOADS + BN / RPL;
  static_assert(LOADS % 8 == 0, "loads split evenly over the waves");
  constexpr int D = LOADS / 8, LA = NBUF - 1;
  static_assert((LA - 1) * D < 64, "vmcnt range");
  constexpr int KC = BK / 32;  // MFMA k chunks per stage
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];  // [NBUF][STAGE]
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wv >> 2, wn = wv & 3;
  const int nks = K / BK;

  const int G = gridDim.x, nx = G < 8 ? G : 8, g = blockIdx.x, x = g % nx, y = g / nx;
  const int Gx = (G - x + nx - 1) / nx;
  const int total = m_tiles * n_tiles;
  const int tx0 = (int)((int64_t)total * x / nx), tx1 = (int)((int64_t)total * (x + 1) / nx);
  const int n_my = tx1 - tx0 > y ? (tx1 - tx0 - y + Gx - 1) / Gx : 0;
  if (n_my == 0) return;
  const int S = n_my * nks;

  // the loads of stage q; past the last stage they repeat it (in bounds, never read)
  const int lrow = lane / UPR, lunit = lane % UPR;
  int ld_q = 0, ld_tile = 0, ld_ks = 0, ld_buf = 0;
  const uint16_t* srcA = nullptr;
  const uint16_t* srcB = nullptr;
  auto aim = [&]() {
    const int t = tx0 + y + ld_tile * Gx, mt = t % m_tiles, nt = t / m_tiles;
    srcA = A + (size_t)mt * BM * lda;
    srcB = B + (size_t)nt * BN * ldb;
    return mt;
  };
  int ld_mt = aim();
  int ld_nt = (tx0 + y) / m_tiles;
  auto issue_one = [&](int d) {
    const int L = wv * D + d;
    const bool isA = L < A_LOADS;
    const int r = (isA ? L : L - A_LOADS) * RPL + lrow;
    const int unit = lunit ^ wide_swizzle<BK>(r);
    const uint16_t* src = isA ? srcA + (size_t)min(r, M - 1 - ld_mt * BM) * lda
                              : srcB + (size_t)min(r, N - 1 - ld_nt * BN) * ldb;
    __builtin_amdgcn_global_load_lds((const void*)(src + ld_ks * BK + unit * 8),
                                     (__attribute__((address_space(3))) void*)(lds + (size_t)ld_buf * STAGE + L * 1024),
                                     16, 0, 0);
  };
  auto advance = [&]() {
    ld_buf = ld_buf + 1 == NBUF ? 0 : ld_buf + 1;
    if (ld_q + 1 < S) {
      ++ld_q;
      if (++ld_ks == nks) {
        ld_ks = 0;
        ++ld_tile;
        ld_mt = aim();
        ld_nt = (tx0 + y + ld_tile * Gx) / m_tiles;
      }
    }
  };
  auto issue = [&]() {
#pragma unroll
    for (int d = 0; d < D; ++d) issue_one(d);
    advance();
  };
  auto sync = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // fragment reads: row l % 16 of a 16-row tile, unit UPR-chunk c: 4c + l / 16
  const int fr = lane & 15, sw = wide_swizzle<BK>(fr);
  int off[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) off[c] = fr * ROWB + (((4 * c + (lane >> 4)) ^ sw) * 16);
  f32x4 acc[MT][NT];
  int rd_buf = 0;
  auto stage = [&](bool first) {
    const unsigned char* a0 = lds + rd_buf * STAGE + wm * MT * 16 * ROWB;
    const unsigned char* b0 = lds + rd_buf * STAGE + A_BYTES + wn * NT * 16 * ROWB;
    rd_buf = rd_buf + 1 == NBUF ? 0 : rd_buf + 1;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      bf16x8 fa[MT], fb[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(b0 + j * 16 * ROWB + off[c]);
#pragma unroll
      for (int i = 0; i < MT; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(a0 + i * 16 * ROWB + off[c]);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = mma(fa[i], fb[j], (first && c == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[i][j]);
      }
    }
  };
  // end of stage q: stage q + 1 in (loads of q + 2 .. q + LA still out), then the barrier
  auto finish = [&]() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((LA - 1) * D) : "memory");
    sync();
  };

  for (int q = 0; q < LA; ++q) issue();
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((LA - 1) * D) : "memory");
  sync();
  for (int i = 0; i < n_my; ++i) {
    issue();
    stage(true);
    finish();
    for (int ks = 1; ks < nks; ++ks) {
      issue();
      stage(false);
      finish();
    }
    const int t = tx0 + y + i * Gx, mt = t % m_tiles, nt = t / m_tiles;
    const int m0 = mt * BM + wm * MT * 16 + (lane >> 4) * 4, n0 = nt * BN + wn * NT * 16 + fr;
    if (mt * BM + BM <= M && nt * BN + BN <= N) {
#pragma unroll
      for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int b = 0; b < NT; ++b) C[(size_t)(m0 + a * 16 + e) * ldc + n0 + b * 16] = acc[a][b][e];
    } else {
#pragma unroll
      for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int b = 0; b < NT; ++b)
            if (m0 + a * 16 + e < M && n0 + b * 16 < N) C[(size_t)(m0 + a * 16 + e) * ldc + n0 + b * 16] = acc[a][b][e];
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
  constexpr int NT = kStreamNT;
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

// LDS beyond 64 KB per workgroup has to be asked for once per kernel and device
static hipError_t allow_lds(const void* fn, size_t bytes) {
  static thread_local const void* done_fn[8];
  static thread_local int done_dev[8] = {-1, -1, -1, -1, -1, -1, -1, -1};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  for (int i = 0; i < 8; ++i)
    if (done_fn[i] == fn && done_dev[i] == dev) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  for (int i = 0; i < 8; ++i)
    if (done_dev[i] < 0) {
      done_fn[i] = fn;
      done_dev[i] = dev;
      break;
    }
  return hipSuccess;
}

template <int MT, int NT>
static hipError_t launch_wide(const uint16_t* A, int lda, const uint16_t* B, int ldb, float* C, int ldc, int M, int N,
                              int K, int cus, hipStream_t s) {
  constexpr int BK = kWideBK, NBUF = kWideNBuf, BM = 2 * MT * 16, BN = 4 * NT * 16;
  constexpr size_t lds = (size_t)NBUF * (BM + BN) * BK * 2;
  static_assert(lds <= 160 * 1024, "LDS of a CU");
  const int m_tiles = (M + BM - 1) / BM, n_tiles = (N + BN - 1) / BN;
  const int64_t total = (int64_t)m_tiles * n_tiles;
  const int grid = total < cus ? (int)total : cus;
  hipError_t e = allow_lds((const void*)gemm_wide<MT, BK, NBUF, NT>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_wide<MT, BK, NBUF, NT>), dim3(grid), dim3(512), lds, s, A, lda, B, ldb, C, ldc, M, N, K, m_tiles,
                     n_tiles);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(int dtype, const void* A, int lda, const void* B, int ldb, float* C, int ldc, int M, int N,
                          int K, bool prefer_tiles, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (N <= 4096 && M <= 4096) {  // few columns and rows: split k inside each workgroup
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
    const int cus = device_cus();
    // whole 256-wide slabs; A, eight 8 KB slabs and the partial sums within the LDS; at least one
    // tile per wave, so that no tile is cut twice.  The block store needs every wave's finished
    // tiles (at most ceil(tiles per workgroup / waves) of them) to fit its registers, and the
    // block ([16][tiles * 16] fp32) to fit the A and slab space.
    constexpr int SW = 8;
    const size_t slds = (size_t)(K / 32) * 64 * 16 + (size_t)SW * 8192;
    if (cus > 0 && K % kR16SlabK == 0 && lda % 8 == 0 && ldb % 8 == 0 && ldb < (1 << 26) &&
        slds + SW * 64 * 16 <= 160 * 1024 && (N + 15) / 16 >= SW * cus) {
      const int per_wg = ((N + 15) / 16 + cus - 1) / cus;
      const bool stage = (per_wg + SW - 1) / SW <= kR16Keep && (size_t)per_wg * 1024 <= slds;
      const void* fn = stage ? (const void*)gemm_rows16_slab<SW, true> : (const void*)gemm_rows16_slab<SW, false>;
      static thread_local int slab_attr_device[2] = {-1, -1};
      int dev = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e != hipSuccess) return e;
      if (slab_attr_device[stage] != dev) {
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(160 * 1024 - SW * 64 * 16));
        if (e != hipSuccess) return e;
        slab_attr_device[stage] = dev;
      }
      if (stage)
        hipLaunchKernelGGL((gemm_rows16_slab<SW, true>), dim3(cus), dim3(64 * SW), slds, s, (const uint16_t*)A, lda,
                           (const uint16_t*)B, ldb, C, ldc, M, N, K);
      else
        hipLaunchKernelGGL((gemm_rows16_slab<SW, false>), dim3(cus), dim3(64 * SW), slds, s, (const uint16_t*)A,
                           lda, (const uint16_t*)B, ldb, C, ldc, M, N, K);
      return hipGetLastError();
    }
    constexpr int WV = kR16Waves;
    const size_t lds = (size_t)((K + 31) / 32) * 64 * 16;
    if (cus > 0 && (N + 15) / 16 >= WV * cus && lds <= 128 * 1024) {
      static thread_local int attr_device = -1;
      int dev = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e != hipSuccess) return e;
      if (attr_device != dev) {
        e = hipFuncSetAttribute((const void*)gemm_rows16<WV, kR16U>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                128 * 1024);
        if (e != hipSuccess) return e;
        attr_device = dev;
      }
      hipLaunchKernelGGL((gemm_rows16<WV, kR16U>), dim3(cus), dim3(64 * WV), lds, s, (const uint16_t*)A, lda,
                         (const uint16_t*)B, ldb, C, ldc, M, N, K);
      return hipGetLastError();
    }
  }
  // Tile shapes by row count (measured at V = 151936): one row tile of 128 or
  // 256 rows takes 320 columns, so that the 475 column tiles need at most two
  // rounds of the CUs (256 columns leave a third, partial round); above 256
  // rows the 256 x 256 tile is faster.
  if (prefer_tiles && M > 16 && K % kWideBK == 0 && lda % 8 == 0 && ldb % 8 == 0) {
    const int cus = device_cus();
    const uint16_t *a16 = (const uint16_t*)A, *b16 = (const uint16_t*)B;
    if (cus > 0 && M > 256) return launch_wide<8, 4>(a16, lda, b16, ldb, C, ldc, M, N, K, cus, s);
    if (cus > 0 && M > 128) return launch_wide<8, 5>(a16, lda, b16, ldb, C, ldc, M, N, K, cus, s);
    if (cus > 0) return launch_wide<4, 5>(a16, lda, b16, ldb, C, ldc, M, N, K, cus, s);
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
