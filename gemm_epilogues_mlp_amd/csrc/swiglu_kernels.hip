// swiglu_kernels.hip -- hand-written gfx950 kernels of the fused SwiGLU MLP GEMM
// Y = SiLU(A W1) (.) (A W2), bf16 in, fp32 accumulate, bf16 out.
//
// Method: gist.science, "Riepilogo Tecnico: Sovrapposizione delle Attivazioni
// a Livello di Tile per l'Inferenza Efficiente di LLM" [RT]:
//   §Metodologia, Kernel-1 ("sync"): per output tile, the Gate product is
//     completed first; SiLU is applied to its register-resident accumulator
//     while the first Up weight tiles are in flight; the Up product follows
//     and the epilogue multiplies and stores.
//   §Metodologia, Kernel-2 ("interleave"): one GEMM over W_fused [K, 2N]
//     (Gate in even, Up in odd columns); the epilogue pairs adjacent
//     accumulator columns, SiLU(even) * odd, and stores N columns.
//   §Definizione del Problema: the unfused baseline (two GEMMs that write
//     Gate and Up to HBM, then a separate activation).
//
// Two kernel families, both built on the MFMA conventions in swiglu_device.hpp:
//
//  * tiled_kernel   LDS-tiled, v_mfma_f32_32x32x16_bf16, 256 threads.  Tiles of
//    A [BM, BK] and of the weights are staged through registers into a
//    double-buffered, row-padded LDS tile (one barrier per K step); the
//    weight tile is transposed to k-contiguous rows on the way in.  For the
//    interleave mode the transposition also separates even (Gate) and odd (Up)
//    columns into two LDS regions, so a lane's Gate and Up accumulators for
//    the same output column sit in the same register of two accumulator sets
//    and the pair-multiply epilogue needs no data exchange.
//
//  * skinny_kernel  split-K weight streaming for small M (decode-sized
//    batches), v_mfma_f32_16x16x32_bf16.  Each lane loads an 8 (k) x 8 (column)
//    block of weights straight from HBM into registers, transposes it there
//    and feeds it to 8 MFMAs; the waves of a workgroup split K and their fp32
//    partial accumulators are reduced through LDS in a fixed order before any
//    SiLU is applied (the activation is nonlinear, so partial sums must be
//    complete and fp32 [RT §Contributi Chiave, item 3 blames bf16 partial
//    accumulation across tiles for the baseline's errors]).  In interleave
//    mode a lane holds 8 consecutive W_fused columns in 8 accumulators, so the
//    pair (2n, 2n+1) is two adjacent accumulators of one lane.
#include "swiglu_device.hpp"
#include "swiglu_internal.h"

namespace swiglu {

enum Mode { MODE_INTERLEAVE = 0, MODE_SYNC = 1, MODE_GEMM = 2 };

// ============================================================================
// LDS-tiled MFMA kernel
// ============================================================================
template <int MODE, int BM, int BNY, int BK, int WGM, int WGN>
struct Tiled {
  static constexpr int kThreads = 256;
  static_assert(WGM * WGN == 4, "four waves per workgroup");
  // weight columns staged per K step
  static constexpr int NC = (MODE == MODE_INTERLEAVE) ? 2 * BNY : BNY;
  static constexpr int WTM = BM / WGM;  // rows per wave
  static constexpr int WTN = BNY / WGN; // output columns per wave
  static constexpr int FM = WTM / 32;
  static constexpr int FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(BK % 16 == 0 && BK >= 16, "BK");
  static constexpr int LDK = BK + 8;  // padded LDS row, elements (16 B pad)
  static constexpr int A_CHUNKS = BM * BK / 8;
  static_assert(A_CHUNKS % kThreads == 0, "A tile must split evenly");
  static constexpr int A_PER_T = A_CHUNKS / kThreads;
  static constexpr int W_BLOCKS = (BK / 8) * (NC / 8);
  static constexpr int W_PER_T = (W_BLOCKS + kThreads - 1) / kThreads;
  static constexpr int LDS_A = BM * LDK;  // elements per stage
  static constexpr int LDS_B = NC * LDK;
  static constexpr int LDS_BYTES = 2 * (LDS_A + LDS_B) * 2;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

template <int MODE, int BM, int BNY, int BK, int WGM, int WGN>
__global__ __launch_bounds__(256) void tiled_kernel(const uint16_t* __restrict__ A,
                                                    const uint16_t* __restrict__ W1,
                                                    const uint16_t* __restrict__ W2,
                                                    uint16_t* __restrict__ Y, int M, int N,
                                                    int K, int group_m) {
  using C = Tiled<MODE, BM, BNY, BK, WGM, WGN>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[C::LDS_BYTES / 2];
  uint16_t* As = smem;                     // [2][BM][LDK]
  uint16_t* Bs = smem + 2 * C::LDS_A;      // [2][NC][LDK]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // ---- tile id: XCD-contiguous ranges, then GROUP_M-major order -------------
  const int ntm = (M + BM - 1) / BM;
  const int ntn = (N + BNY - 1) / BNY;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = group_m * ntn;
  const int grp = t / per_group;
  const int first_m = grp * group_m;
  const int gsz = min(ntm - first_m, group_m);
  const int tm = first_m + (t % per_group) % gsz;
  const int tn = (t % per_group) / gsz;
  const int m0 = tm * BM;
  const int n0 = tn * BNY;  // first output column

  const int nk = (K + BK - 1) / BK;
  const int total = (MODE == MODE_SYNC) ? 2 * nk : nk;

  // ---- global -> register staging ------------------------------------------
  u32x4 ra[C::A_PER_T];
  u32x4 rw[C::W_PER_T][8];

  auto gload = [&](int it) {
    const int kt = (MODE == MODE_SYNC) ? (it < nk ? it : it - nk) : it;
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int idx = tid + C::kThreads * i;
      const int row = idx / (BK / 8), kc = idx % (BK / 8);
      const int gm = m0 + row, gk = k0 + kc * 8;
      ra[i] = (gm < M && gk < K) ? load16(A + (size_t)gm * K + gk) : u32x4{0, 0, 0, 0};
    }
    const uint16_t* W;
    int ldw, ncols, cbase;
    if (MODE == MODE_INTERLEAVE) {
      W = W1, ldw = 2 * N, ncols = 2 * N, cbase = 2 * n0;
    } else if (MODE == MODE_SYNC) {
      W = (it < nk) ? W1 : W2, ldw = N, ncols = N, cbase = n0;
    } else {
      W = W1, ldw = N, ncols = N, cbase = n0;
    }
#pragma unroll
    for (int i = 0; i < C::W_PER_T; ++i) {
      const int idx = tid + C::kThreads * i;
      const int kb = idx / (C::NC / 8), nb = idx % (C::NC / 8);
      const int col = cbase + nb * 8;
      const int gk = k0 + kb * 8;
      const bool ok = (idx < C::W_BLOCKS) && gk < K && col < ncols;
      const uint16_t* p = W + (size_t)gk * ldw + col;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        rw[i][r] = ok ? load16(p + (size_t)r * ldw) : u32x4{0, 0, 0, 0};
    }
  };

  auto swrite = [&](int buf) {
    uint16_t* as = As + buf * C::LDS_A;
    uint16_t* bs = Bs + buf * C::LDS_B;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int idx = tid + C::kThreads * i;
      const int row = idx / (BK / 8), kc = idx % (BK / 8);
      *reinterpret_cast<u32x4*>(as + row * C::LDK + kc * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::W_PER_T; ++i) {
      const int idx = tid + C::kThreads * i;
      if (idx < C::W_BLOCKS) {
        const int kb = idx / (C::NC / 8), nb = idx % (C::NC / 8);
        u32x4 col[8];
        transpose8x8(rw[i], col);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int lc = nb * 8 + c;
          // interleave: even W_fused column -> Gate row lc/2, odd -> Up row BNY + lc/2
          const int lrow = (MODE == MODE_INTERLEAVE) ? ((lc & 1) * BNY + (lc >> 1)) : lc;
          *reinterpret_cast<u32x4*>(bs + lrow * C::LDK + kb * 8) = col[c];
        }
      }
    }
  };

  f32x16 acc0[C::FM][C::FN];
  f32x16 acc1[(MODE == MODE_GEMM) ? 1 : C::FM][(MODE == MODE_GEMM) ? 1 : C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      acc0[i][j] = f32x16{};
      if (MODE != MODE_GEMM) acc1[i][j] = f32x16{};
    }

  // per-lane fragment coordinates
  const int frow = lane & 31;        // row (A) or column (B) inside a 32 block
  const int fk = (lane >> 5) * 8;    // k offset inside a 16-deep step

  auto compute = [&](int buf, int phase) {
    const uint16_t* as = As + buf * C::LDS_A;
    const uint16_t* bs = Bs + buf * C::LDS_B;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      u32x4 af[C::FM], bf[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(as + (wm * C::WTM + i * 32 + frow) * C::LDK + kk + fk);
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(bs + (wn * C::WTN + j * 32 + frow) * C::LDK + kk + fk);
      if (MODE == MODE_INTERLEAVE) {
        u32x4 bu[C::FN];
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          bu[j] = *reinterpret_cast<const u32x4*>(bs + (BNY + wn * C::WTN + j * 32 + frow) * C::LDK + kk + fk);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            acc0[i][j] = mfma32(af[i], bf[j], acc0[i][j]);
            acc1[i][j] = mfma32(af[i], bu[j], acc1[i][j]);
          }
      } else if (MODE == MODE_SYNC && phase != 0) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) acc1[i][j] = mfma32(af[i], bf[j], acc1[i][j]);
      } else {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) acc0[i][j] = mfma32(af[i], bf[j], acc0[i][j]);
      }
    }
  };

  // ---- main loop: one barrier per K step -----------------------------------
  if (total > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();
  if (total > 1) gload(1);
  for (int it = 0; it < total; ++it) {
    const int cur = it & 1;
    const int phase = (MODE == MODE_SYNC && it >= nk) ? 1 : 0;
    compute(cur, phase);
    if (it + 1 < total) swrite(cur ^ 1);
    if (it + 2 < total) gload(it + 2);
    if (MODE == MODE_SYNC && it == nk - 1) {
      // Gate finished: SiLU on the register-resident Gate accumulator while
      // the first Up weight tiles are in flight.
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc0[i][j][r] = silu(acc0[i][j][r]);
    }
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------
  const int col_in = lane & 31;
  const int row_q = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int col = n0 + wn * C::WTN + j * 32 + col_in;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * C::WTM + i * 32 + (r >> 2) * 8 + row_q + (r & 3);
        float v;
        if (MODE == MODE_INTERLEAVE) v = silu(acc0[i][j][r]) * acc1[i][j][r];
        else if (MODE == MODE_SYNC) v = acc0[i][j][r] * acc1[i][j][r];
        else v = acc0[i][j][r];
        if (row < M && col < N) Y[(size_t)row * N + col] = bf16_bits(v);
      }
    }
}

// ============================================================================
// Split-K weight-streaming kernel for small M
// ============================================================================
// A workgroup owns one slab of 128 weight columns and MT*16 rows of A; its NW
// waves split the K steps (32 deep) into contiguous ranges.
//   interleave: W_fused columns [128 s, 128 s + 128)  -> Y columns [64 s, +64)
//   sync      : W1 and W2 columns [64 s, 64 s + 64)   -> Y columns [64 s, +64)
//               (lane loads 4 Gate and 4 Up columns; with K split across waves
//               the activation can only follow the reduction, so both
//               weights stream in one K loop)
//   gemm      : W1 columns [128 s, +128)              -> G columns, same range
template <int MODE, int MT, int NW>
struct Skinny {
  static constexpr int kThreads = 64 * NW;
  static constexpr int LDS_BYTES = NW * MT * 8 * 64 * 16;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static constexpr int SLAB_Y = (MODE == MODE_GEMM) ? 128 : 64;  // output cols per slab
};

template <int MODE, int MT>
__device__ __forceinline__ void skinny_load(const uint16_t* __restrict__ A,
                                            const uint16_t* __restrict__ W1,
                                            const uint16_t* __restrict__ W2, int M, int N,
                                            int K, int m0, int slab, int lane, int step,
                                            u32x4 (&rows)[8], u32x4 (&af)[MT]) {
  const int cg = lane & 15;
  const int k = step * 32 + (lane >> 4) * 8;
  const bool kin = k < K;  // K % 8 == 0: the 8 rows are all in or all out
  if (MODE == MODE_SYNC) {
    const int c = slab * 64 + cg * 4;
    const bool ok = kin && c < N;
    const uint16_t* p1 = W1 + (size_t)k * N + c;
    const uint16_t* p2 = W2 + (size_t)k * N + c;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      u32x2 g = ok ? load8(p1 + (size_t)r * N) : u32x2{0, 0};
      u32x2 u = ok ? load8(p2 + (size_t)r * N) : u32x2{0, 0};
      rows[r] = u32x4{g[0], g[1], u[0], u[1]};
    }
  } else {
    const int ld = (MODE == MODE_INTERLEAVE) ? 2 * N : N;
    const int c = slab * 128 + cg * 8;
    const bool ok = kin && c < ld;
    const uint16_t* p = W1 + (size_t)k * ld + c;
#pragma unroll
    for (int r = 0; r < 8; ++r) rows[r] = ok ? load16(p + (size_t)r * ld) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + mt * 16 + (lane & 15);
    af[mt] = (kin && m < M) ? load16(A + (size_t)m * K + k) : u32x4{0, 0, 0, 0};
  }
}

template <int MODE, int MT, int NW>
__global__ __launch_bounds__(64 * NW) void skinny_kernel(const uint16_t* __restrict__ A,
                                                         const uint16_t* __restrict__ W1,
                                                         const uint16_t* __restrict__ W2,
                                                         uint16_t* __restrict__ Y, int M, int N,
                                                         int K) {
  using C = Skinny<MODE, MT, NW>;
  __shared__ __attribute__((aligned(16))) f32x4 red[NW * MT * 8 * 64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nslab = gridDim.x;
  const int slab = xcd_remap(blockIdx.x, nslab);
  const int m0 = blockIdx.y * MT * 16;

  const int nsteps = (K + 31) / 32;
  const int per = (nsteps + NW - 1) / NW;
  const int s_begin = wave * per;
  const int s_end = min(nsteps, s_begin + per);

  f32x4 acc[MT][8];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[mt][c] = f32x4{};

  auto mma = [&](const u32x4 (&rows)[8], const u32x4 (&af)[MT]) {
    u32x4 col[8];
    transpose8x8(rows, col);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt][c] = mfma16(af[mt], col[c], acc[mt][c]);
  };

  // two register sets: the loads of step s+1 are in flight while step s computes
  u32x4 r0[8], r1[8];
  u32x4 a0[MT], a1[MT];
  int s = s_begin;
  if (s < s_end) skinny_load<MODE, MT>(A, W1, W2, M, N, K, m0, slab, lane, s, r0, a0);
  while (s < s_end) {
    if (s + 1 < s_end) skinny_load<MODE, MT>(A, W1, W2, M, N, K, m0, slab, lane, s + 1, r1, a1);
    mma(r0, a0);
    if (s + 1 >= s_end) break;
    if (s + 2 < s_end) skinny_load<MODE, MT>(A, W1, W2, M, N, K, m0, slab, lane, s + 2, r0, a0);
    mma(r1, a1);
    s += 2;
  }

  // ---- split-K reduction through LDS (fixed order: wave 0, 1, ..., NW-1) ----
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int c = 0; c < 8; ++c) red[((wave * MT + mt) * 8 + c) * 64 + lane] = acc[mt][c];
  __syncthreads();

  const int cg = lane & 15;
  const int rq = (lane >> 4) * 4;
  for (int mt = wave; mt < MT; mt += NW) {
    f32x4 v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      v[c] = red[(mt * 8 + c) * 64 + lane];
      for (int w = 1; w < NW; ++w) v[c] += red[((w * MT + mt) * 8 + c) * 64 + lane];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + mt * 16 + rq + r;
      if (row >= M) continue;
      if (MODE == MODE_GEMM) {
        const int col = slab * 128 + cg * 8;
        if (col < N) {
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(v[2 * q][r], v[2 * q + 1][r]);
          *reinterpret_cast<u32x4*>(Y + (size_t)row * N + col) = o;
        }
      } else {
        const int col = slab * 64 + cg * 4;
        if (col < N) {
          float y[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // interleave: adjacent accumulators (2q Gate, 2q+1 Up);
            // sync: accumulator q is Gate, q+4 the matching Up column
            const float g = (MODE == MODE_INTERLEAVE) ? v[2 * q][r] : v[q][r];
            const float u = (MODE == MODE_INTERLEAVE) ? v[2 * q + 1][r] : v[q + 4][r];
            y[q] = silu(g) * u;
          }
          u32x2 o{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
          *reinterpret_cast<u32x2*>(Y + (size_t)row * N + col) = o;
        }
      }
    }
  }
}

// ============================================================================
// Unfused baseline element-wise gate and the W_fused pack kernel
// ============================================================================
// Y = bf16(SiLU(G) * U) element-wise, G and U bf16, fp32 arithmetic; 8
// elements (16 B) per thread per iteration, grid-stride.
__global__ __launch_bounds__(256) void gate_kernel(const uint16_t* __restrict__ G,
                                                   const uint16_t* __restrict__ U,
                                                   uint16_t* __restrict__ Y, size_t n8) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (size_t)gridDim.x * blockDim.x) {
    const u32x4 g = load16(G + i * 8);
    const u32x4 u = load16(U + i * 8);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float g0 = bf16_to_float((uint16_t)(g[q] & 0xffffu));
      const float g1 = bf16_to_float((uint16_t)(g[q] >> 16));
      const float u0 = bf16_to_float((uint16_t)(u[q] & 0xffffu));
      const float u1 = bf16_to_float((uint16_t)(u[q] >> 16));
      o[q] = pack_bf16x2(silu(g0) * u0, silu(g1) * u1);
    }
    *reinterpret_cast<u32x4*>(Y + i * 8) = o;
  }
}

// W_fused[k, 2n] = W1[k, n], W_fused[k, 2n+1] = W2[k, n]; a thread moves 8
// columns of one row (16 B from each source, 32 B out).
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ W1,
                                                   const uint16_t* __restrict__ W2,
                                                   uint16_t* __restrict__ WF, size_t n8) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (size_t)gridDim.x * blockDim.x) {
    const u32x4 a = load16(W1 + i * 8);
    const u32x4 b = load16(W2 + i * 8);
    u32x4 lo, hi;
    lo[0] = __builtin_amdgcn_perm(b[0], a[0], 0x05040100u);
    lo[1] = __builtin_amdgcn_perm(b[0], a[0], 0x07060302u);
    lo[2] = __builtin_amdgcn_perm(b[1], a[1], 0x05040100u);
    lo[3] = __builtin_amdgcn_perm(b[1], a[1], 0x07060302u);
    hi[0] = __builtin_amdgcn_perm(b[2], a[2], 0x05040100u);
    hi[1] = __builtin_amdgcn_perm(b[2], a[2], 0x07060302u);
    hi[2] = __builtin_amdgcn_perm(b[3], a[3], 0x05040100u);
    hi[3] = __builtin_amdgcn_perm(b[3], a[3], 0x07060302u);
    // the 8 source columns of row k start at n = 8*(i % (N/8)); W_fused row k
    // is twice as long, so output index = 2 * input index
    *reinterpret_cast<u32x4*>(WF + i * 16) = lo;
    *reinterpret_cast<u32x4*>(WF + i * 16 + 8) = hi;
  }
}

// ============================================================================
// Configuration list and launchers
// ============================================================================
template <int MODE, int BM, int BNY, int BK, int WGM, int WGN>
static hipError_t launch_tiled(const LaunchArgs& a) {
  using C = Tiled<MODE, BM, BNY, BK, WGM, WGN>;
  const int ntm = (a.M + BM - 1) / BM, ntn = (a.N + BNY - 1) / BNY;
  const long long nwg = (long long)ntm * ntn;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  int group_m = a.group_m > 0 ? a.group_m : 8;
  if (group_m > ntm) group_m = ntm;
  hipLaunchKernelGGL((tiled_kernel<MODE, BM, BNY, BK, WGM, WGN>), dim3((unsigned)nwg),
                     dim3(C::kThreads), 0, a.stream, a.A, a.W1, a.W2, a.Y, a.M, a.N, a.K,
                     group_m);
  return hipGetLastError();
}

template <int MODE, int MT, int NW>
static hipError_t launch_skinny(const LaunchArgs& a) {
  using C = Skinny<MODE, MT, NW>;
  const long long nslab = (a.N + C::SLAB_Y - 1) / C::SLAB_Y;
  const long long nmb = (a.M + MT * 16 - 1) / (MT * 16);
  if (nslab <= 0 || nmb <= 0) return hipSuccess;
  if (nslab > 0x7fffffffLL || nmb > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((skinny_kernel<MODE, MT, NW>), dim3((unsigned)nslab, (unsigned)nmb),
                     dim3(C::kThreads), 0, a.stream, a.A, a.W1, a.W2, a.Y, a.M, a.N, a.K);
  return hipGetLastError();
}

#define TILED(mode, v, bm, bn, bk, wgm, wgn)                                               \
  {v, 0, bm, bn, bk, 4, 1, Tiled<mode, bm, bn, bk, wgm, wgn>::LDS_BYTES,                  \
   &launch_tiled<mode, bm, bn, bk, wgm, wgn>}
#define SKINNY(mode, v, mt, nw)                                                            \
  {v, 1, (mt) * 16, Skinny<mode, mt, nw>::SLAB_Y, 32, nw, nw, Skinny<mode, mt, nw>::LDS_BYTES, \
   &launch_skinny<mode, mt, nw>}

static const KernelConfig kConfigs[] = {
    // ---- interleave (Kernel-2 family) --------------------------------------
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 256, 128, 64, 2, 2),  // 0
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 128, 128, 64, 2, 2),  // 1
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 128, 64, 64, 2, 2),   // 2
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 64, 64, 64, 2, 2),    // 3
    SKINNY(MODE_INTERLEAVE, VAR_INTERLEAVE, 1, 8),               // 4
    SKINNY(MODE_INTERLEAVE, VAR_INTERLEAVE, 2, 8),               // 5
    SKINNY(MODE_INTERLEAVE, VAR_INTERLEAVE, 4, 4),               // 6
    // ---- sync (Kernel-1 family) --------------------------------------------
    TILED(MODE_SYNC, VAR_SYNC, 256, 128, 64, 2, 2),              // 7
    TILED(MODE_SYNC, VAR_SYNC, 128, 128, 64, 2, 2),              // 8
    TILED(MODE_SYNC, VAR_SYNC, 128, 64, 64, 2, 2),               // 9
    TILED(MODE_SYNC, VAR_SYNC, 64, 64, 64, 2, 2),                // 10
    SKINNY(MODE_SYNC, VAR_SYNC, 1, 8),                           // 11
    SKINNY(MODE_SYNC, VAR_SYNC, 2, 8),                           // 12
    SKINNY(MODE_SYNC, VAR_SYNC, 4, 4),                           // 13
    // ---- plain GEMM for the unfused baseline -------------------------------
    TILED(MODE_GEMM, VAR_GEMM, 256, 256, 64, 2, 2),              // 14
    TILED(MODE_GEMM, VAR_GEMM, 256, 128, 64, 2, 2),              // 15
    TILED(MODE_GEMM, VAR_GEMM, 128, 128, 64, 2, 2),              // 16
    TILED(MODE_GEMM, VAR_GEMM, 64, 64, 64, 2, 2),                // 17
    SKINNY(MODE_GEMM, VAR_GEMM, 1, 8),                           // 18
    SKINNY(MODE_GEMM, VAR_GEMM, 2, 8),                           // 19
    SKINNY(MODE_GEMM, VAR_GEMM, 4, 4),                           // 20
};

int config_count() { return (int)(sizeof(kConfigs) / sizeof(kConfigs[0])); }
const KernelConfig* config_at(int id) {
  return (id >= 0 && id < config_count()) ? &kConfigs[id] : nullptr;
}

hipError_t launch_gate(const uint16_t* G, const uint16_t* U, uint16_t* Y, size_t n,
                       hipStream_t stream, int cu_count) {
  const size_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  size_t blocks = (n8 + 255) / 256;
  const size_t cap = (size_t)(cu_count > 0 ? cu_count : 256) * 8;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(gate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, G, U, Y, n8);
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* W1, const uint16_t* W2, uint16_t* WF, size_t n,
                       hipStream_t stream, int cu_count) {
  const size_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  size_t blocks = (n8 + 255) / 256;
  const size_t cap = (size_t)(cu_count > 0 ? cu_count : 256) * 8;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W1, W2, WF, n8);
  return hipGetLastError();
}

}  // namespace swiglu
