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
// Kernel families, all on the MFMA conventions in swiglu_device.hpp (each is
// described in detail where it is defined):
//
//  * tiled_kernel / tiled_split_kernel / tiled_persist_kernel  LDS-tiled bf16,
//    v_mfma_f32_32x32x16_bf16, 4 or 8 waves.  A and weight k-tiles go from HBM
//    straight into a ring of LDS stages by DMA; weight fragments are read with
//    the transposing LDS read; the MFMA computes D^T = W^T A^T so that a Gate
//    / Up pair of the interleave mode sits in two adjacent registers of one
//    lane.  Interleave, sync and plain-GEMM (unfused baseline) modes.  The
//    split launch runs a short last round as quarter tiles; the persistent one
//    keeps one workgroup per CU looping over tiles, the next tile's loads
//    issued under the current tile's last K steps (Kernel-2's overlap).
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
//
//  * packed_kernel  the same streaming on W_fused stored once in MFMA
//    fragment order: 1 KB contiguous per load, no transposition.
//    packed_mixed_kernel runs whole slabs and quarter slabs in one launch, so
//    that slab counts a little above a whole number per CU stay balanced;
//    packed_splitk_kernel also splits K over workgroups (decode shapes with
//    few slabs): fp32 partials handed to the last workgroup of each slab part,
//    which reduces them in K order before SiLU.
//
//  * f8_kernel / f8_split_kernel / f8_skinny_kernel / f8_packed_kernel  FP8
//    (E4M3) inputs on the scaled MFMAs, LDS-tiled and streaming, in both
//    orders; MX modes of the tile (both orders) and mx_packed_kernel for
//    MXFP8 (E8M0 block scales applied by the MFMA).
//
//  * element-wise kernels: the unfused gate, the weight packs and the FP8 /
//    MX quantisers.
#include "swiglu_device.hpp"
#include "swiglu_internal.h"

#include <tuple>
#include <type_traits>
#include <utility>

namespace swiglu {

// MODE_MX / MODE_MX_SYNC: the interleave and the sync order on MXFP8 inputs
// (FP8 tile kernel only).  MODE_PAIR: the sync family's output tile on W1 and
// W2 as stored, with the Gate and Up GEMMs run by two groups of waves over the
// same A k-tiles (bf16 tile kernel only).
enum Mode {
  MODE_INTERLEAVE = 0, MODE_SYNC = 1, MODE_GEMM = 2, MODE_MX = 3, MODE_MX_SYNC = 4, MODE_PAIR = 5
};

// ============================================================================
// LDS-tiled MFMA kernel
// ============================================================================
// One workgroup (4 waves) computes BM rows of A against BNW weight columns
// (interleave: BNW W_fused columns = BNW/2 Y columns; sync: BNW columns of W1
// and then of W2; gemm: BNW columns of one weight).  Each K step of depth BK
// moves A[BM, BK] and W[BK, BNW] from HBM into one of STAGES LDS buffers by
// direct DMA (buffer_load ... lds, no registers), STAGES-1 steps ahead of the
// MFMAs, with one barrier per K step.  Rows, columns and k outside the tensors
// arrive as zeros (buffer loads past the resource size return 0).
//
// Orientation: the MFMA computes D^T = W^T A^T.  Its first source is a weight
// fragment (32 weight columns x 16 k) read with the transposing LDS read from
// the n-contiguous weight tile; its second is an activation fragment (32 rows
// of A x 16 k, one ds_read_b128).  A lane then holds one row of A and, per
// accumulator, four runs of 4 consecutive weight columns in 4 consecutive
// registers: the interleave pair (Gate column 2n, Up column 2n+1) is two
// adjacent registers of one lane, and the pair-multiply epilogue is local.
//
// LDS layouts (16-byte chunks, XOR-swizzled so that the fragment reads are
// free of bank conflicts):
//   A stage  [BM][BK]   row-major, chunk c of row r stored at c ^ a_swz(r)
//   W stage  [BK][BNW]  row-major, chunk c of row k stored at c ^ w_swz(k)
template <int MODE, int BM, int BNW, int BK, int STAGES, int WGM, int WGN>
struct Tiled {
  static constexpr int kWaves = WGM * WGN;
  static_assert(kWaves == 4 || kWaves == 8, "four waves (one per SIMD) or eight (two per SIMD)");
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BNY =
      (MODE == MODE_INTERLEAVE || MODE == MODE_PAIR) ? BNW / 2 : BNW;  // output columns
  static constexpr int WTM = BM / WGM;   // A rows per wave
  static constexpr int WTW = BNW / WGN;  // weight columns per wave
  static constexpr int FA = WTM / 32;    // 32-row blocks of A per wave
  static constexpr int FW = WTW / 32;    // 32-column blocks of W per wave
  static_assert(FA >= 1 && FW >= 1 && WTM % 32 == 0 && WTW % 32 == 0, "wave tile");
  static constexpr int NACC = (MODE == MODE_SYNC) ? 2 : 1;
  static constexpr int NSUB = BK / 16;
  static_assert(BK % 32 == 0, "BK: an even number of 16-deep MFMA steps");
  static constexpr int ACH = BK / 8;     // 16-byte chunks per A row of a stage
  static_assert(ACH == 4 || ACH == 8, "A swizzle covers 4 or 8 chunks");
  static constexpr int WCH = BNW / 8;    // 16-byte chunks per weight row
  static_assert(WCH % 8 == 0 && WCH <= 64, "W swizzle stays inside groups of 8 chunks");
  // A pair tile stores its weight stage as two parts, [BK][BNY] of W1 and
  // then [BK][BNY] of W2, so that every DMA instruction of a wave reads one
  // tensor (the buffer resource is wave-uniform).
  static constexpr int WPARTS = (MODE == MODE_PAIR) ? 2 : 1;
  static constexpr int WCHP = WCH / WPARTS;       // chunks per weight row of a part
  static constexpr int PART_COLS = BNW / WPARTS;  // weight columns per part
  static constexpr int PART_BYTES = BK * PART_COLS * 2;
  static_assert(WCHP % 8 == 0, "W swizzle works on aligned groups of 8 chunks of a part");
  static_assert((BK * WCHP) % 64 == 0, "a wave's 64 weight chunks lie in one part");
  static_assert(MODE != MODE_PAIR || (PART_COLS % WTW == 0 && WGN % 2 == 0),
                "pair tile: each wave's weight columns lie in one part, half the waves each");
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int W_BYTES = BK * BNW * 2;
  static constexpr int STAGE_BYTES = A_BYTES + W_BYTES;
  // DMA instructions per thread (a whole wave without a chunk of its own in
  // the last round loads zeros into a junk slot, so that every wave issues
  // the same number of loads per step and the vmcnt accounting stays uniform)
  static constexpr int A_CHUNKS = BM * ACH, W_CHUNKS = BK * WCH;
  static_assert(A_CHUNKS % 64 == 0 && W_CHUNKS % 64 == 0, "whole waves of chunks");
  static constexpr int A_LOADS = (A_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int W_LOADS = (W_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int LOADS = A_LOADS + W_LOADS;
  static_assert(STAGES >= 2 && LOADS * (STAGES - 2) + LOADS / 2 <= 63, "vmcnt range");
  static constexpr int YLD = BNY + 8;    // padded row of the output staging tile
  // pair tile: the Gate waves hand SiLU(Gate) to the Up waves as fp32 [BM][SLD]
  static constexpr int SLD = BNY + 4;
  static constexpr int Y_BYTES = (MODE == MODE_PAIR) ? BM * SLD * 4 : BM * YLD * 2;
  // 1 KB slot for zero DMA, allocated only when some wave can lack a chunk
  static constexpr bool NEED_JUNK = A_CHUNKS % kThreads != 0 || W_CHUNKS % kThreads != 0;
  static constexpr int JUNK = STAGES * STAGE_BYTES;
  static constexpr int RING_END = JUNK + (NEED_JUNK ? 1024 : 0);
  static constexpr int LDS_BYTES = RING_END > Y_BYTES ? RING_END : Y_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(WCH % 8 == 0, "W swizzle works on aligned groups of 8 chunks");

  // Swizzles: a fragment read touches 16 B per lane; lanes that the LDS
  // serves together (8 lanes per 128 B, or 16 per 256 B) must hit distinct
  // 16-byte bank groups.  A reads take 32 consecutive rows at one logical
  // chunk; W transposing reads take 4 consecutive k rows at 2 (16-lane group)
  // or 4 (32 lanes) consecutive chunks.
  __host__ __device__ static constexpr int a_swz(int row) {
    if (ACH == 8) return (row ^ (row >> 3)) & 7;  // 128 B rows
    return (((row >> 2) & 1) << 1) | (((row >> 1) ^ (row >> 3)) & 1);  // 64 B rows
  }
  // chunk XOR 2*g: the four rows of a 16-lane group land in distinct 32 B
  // slots of 128 B, and together with the neighbouring group in distinct
  // slots of 256 B.  Rows that are an odd multiple of 128 B alternate halves
  // of 256 B by themselves, so g = k % 4 suffices there; rows a multiple of
  // 256 B all start at the same bank and take g = 0, 3, 5, 6 for k % 4 = 0..3.
  __host__ __device__ static constexpr int w_swz(int row) {
    if ((WCHP / 8) % 2 == 1) return (row & 3) << 1;  // rows an odd multiple of 128 B
    return ((0x6530 >> (4 * (row & 3))) & 0xf) << 1;
  }
  // every swizzle must permute the chunks of its own row (checked at compile
  // time for each instantiated tile: a swizzle that left the row would read
  // or write another row's data)
  static constexpr bool swizzles_permute_rows() {
    for (int r = 0; r < 16; ++r) {
      unsigned long long a_seen = 0, w_seen = 0;
      for (int c = 0; c < ACH; ++c) a_seen |= 1ull << (c ^ a_swz(r));
      for (int c = 0; c < WCHP; ++c) {
        const int x = c ^ w_swz(r);
        if (x < 0 || x >= WCHP) return false;
        w_seen |= 1ull << x;
      }
      if (a_seen != (1ull << ACH) - 1 || w_seen != (WCHP >= 64 ? ~0ull : (1ull << WCHP) - 1))
        return false;
    }
    return true;
  }
};


// Position of tile t in the launch order: GROUP_M bands of tile rows, and
// within a band column-major, so that the workgroups running together share
// weight columns and rows of A.
__device__ __forceinline__ void tile_of(int t, int ntm, int ntn, int group_m, int& tm, int& tn) {
  const int per_group = group_m * ntn;
  const int first_m = t / per_group * group_m;
  const int gsz = min(ntm - first_m, group_m);
  tm = first_m + (t % per_group) % gsz;
  tn = (t % per_group) / gsz;
}

// One output tile: rows [m0, m0 + BM) of A against weight columns
// [tn BNW, (tn + 1) BNW), i.e. output columns [tn BNY, (tn + 1) BNY).
// N: output columns of the problem; ldw, ldy: row strides (elements) of the
// weights and of Y.  smem: the workgroup's LDS (at least C::LDS_BYTES).
template <int MODE, int BM, int BNW, int BK, int STAGES, int WGM, int WGN>
__device__ __forceinline__ void tiled_tile(const uint16_t* __restrict__ A,
                                           const uint16_t* __restrict__ W1,
                                           const uint16_t* __restrict__ W2,
                                           uint16_t* __restrict__ Y, int M, int N, int K,
                                           int ldw, int ldy, int m0, int tn, uint8_t* smem) {
  using C = Tiled<MODE, BM, BNW, BK, STAGES, WGM, WGN>;
  static_assert(C::swizzles_permute_rows(), "LDS swizzle is not a permutation of a row");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int y0 = tn * C::BNY;
  // first weight column (of W_fused, of W1 and W2, or of W)
  const int wc0 = (MODE == MODE_PAIR) ? y0 : tn * BNW;

  // K steps.  Step `it` always uses stage it % STAGES and the main loop is
  // unrolled over the stage ring, so every stage offset is a compile-time
  // constant.  The sync variant runs the K steps twice (Gate, then Up); its
  // Gate phase is padded with zero-filled steps to a ring boundary (nk0) so
  // that the Up phase starts on stage 0.
  const int nk = (K + BK - 1) / BK;
  const int nk0 = (MODE == MODE_SYNC) ? (nk + STAGES - 1) / STAGES * STAGES : nk;
  const int total = (MODE == MODE_SYNC) ? nk0 + nk : nk;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave id in an SGPR

  // ---- DMA of one K step into a stage ----------------------------------------
  // Per-thread parts of the byte offsets do not change with k.  A chunk of A
  // is zero-filled if its row or its k is out of range; a weight chunk if its
  // column is (rows past K lie past the end of the weight buffer, so the
  // buffer bound zero-fills them by itself).
  const int wcols = (MODE == MODE_INTERLEAVE) ? 2 * N : N;  // weight columns in range
  const uint32_t wbytes = K > 0 ? (uint32_t)(((size_t)(K - 1) * ldw + wcols) * 2) : 0u;
  const i32x4 rsA = make_rsrc(A, (uint32_t)((size_t)M * K * 2));
  const i32x4 rsW1 = make_rsrc(W1, wbytes);
  const i32x4 rsW2 =
      (MODE == MODE_SYNC || MODE == MODE_PAIR) ? make_rsrc(W2, wbytes) : rsW1;
  const uint32_t lds0 = lds_addr(smem);

  uint32_t a_off[C::A_LOADS];
  int a_k[C::A_LOADS];  // k of the chunk within the step, or a huge value if the row is out
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int p = tid + C::kThreads * i;
    const int row = p / C::ACH;
    const int c = (p % C::ACH) ^ C::a_swz(row);
    a_off[i] = (uint32_t)((m0 + row) * K + c * 8) * 2u;
    a_k[i] = (m0 + row < M) ? c * 8 : 0x3fffffff;
  }
  uint32_t w_off[C::W_LOADS];  // kOutOfRange-based if the column is out of range
#pragma unroll
  for (int i = 0; i < C::W_LOADS; ++i) {
    const int p = (tid + C::kThreads * i) % (BK * C::WCHP);  // chunk within its part
    const int row = p / C::WCHP;
    const int c = (p % C::WCHP) ^ C::w_swz(row);
    w_off[i] = (wc0 + c * 8 < wcols) ? (uint32_t)(row * ldw + wc0 + c * 8) * 2u : kOutOfRange;
  }

  // DMA instruction q (A chunks first, then W chunks) of K step `it` into
  // stage ST.  k0 is capped at K for steps past the end, which keeps every
  // offset below 2^32 and out of range.
  auto dma = [&](int it, auto st_c, int q) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    const bool up = MODE == MODE_SYNC && it >= nk0;
    const int kt = up ? it - nk0 : it;
    const int k0 = (it < total && kt < nk) ? kt * BK : K;
    const uint32_t sbase = lds0 + ST * C::STAGE_BYTES;
    if (q < C::A_LOADS) {
      const int p0 = C::kThreads * q + 64 * wave_u;  // first chunk of this wave
      const bool own = p0 < C::A_CHUNKS;
      const uint32_t off =
          (own && k0 + a_k[q] < K) ? a_off[q] + (uint32_t)k0 * 2u : kOutOfRange;
      lds_dma16(own ? sbase + p0 * 16 : lds0 + C::JUNK, off, rsA);
    } else {
      const int i = q - C::A_LOADS;
      const int p0 = C::kThreads * i + 64 * wave_u;
      const bool own = p0 < C::W_CHUNKS;
      const uint32_t off = own ? w_off[i] + (uint32_t)k0 * (uint32_t)ldw * 2u : kOutOfRange;
      // the W2 part of a pair stage: this wave's chunks all lie in one part
      const bool w2 = up || (MODE == MODE_PAIR && p0 >= BK * C::WCHP);
      lds_dma16(own ? sbase + C::A_BYTES + p0 * 16 : lds0 + C::JUNK, off, w2 ? rsW2 : rsW1);
    }
  };

  // ---- fragments ---------------------------------------------------------------
  // weight fragment: lane l -> weight column 32-block + l%32, k = 8*(l/32)+[0,8)
  const int g16 = lane >> 4, s16 = lane & 15;
  const int w_row = 8 * (g16 >> 1) + (s16 >> 2);                   // + kk, + 4 for 2nd read
  const int w_col = wn * C::WTW + 16 * (g16 & 1) + 4 * (s16 & 3);  // + 32 fw
  // activation fragment: lane l -> A row 32-block + l%32, k = 8*(l/32)+[0,8)
  const int a_row = wm * C::WTM + (lane & 31);                      // + 32 fa
  const int a_chk = lane >> 5;                                     // + kk/8
  constexpr int NFRAG = 2 * C::FW + C::FA;  // LDS reads per sub-step

  u32x4 wf[2][C::FW], af[2][C::FA];
  // fragment read r of sub-step `sub` of stage ST (r < 2 FW: half r%2 of
  // weight block r/2; otherwise A block r - 2 FW)
  auto frag = [&](auto st_c, int sub, int fb, int r) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    const uint8_t* st = smem + ST * C::STAGE_BYTES;
    const int kk = sub * 16;
    if (r < 2 * C::FW) {
      const int fw = r >> 1, h = r & 1;
      const int wcol = w_col + fw * 32;
      const int part = (C::WPARTS == 1) ? 0 : wcol / C::PART_COLS;
      const int col = wcol - part * C::PART_COLS;
      const int row = kk + w_row + 4 * h;
      const int chunk = (col >> 3) ^ C::w_swz(row);
      const u32x2 v = lds_read_tr16(st + C::A_BYTES + part * C::PART_BYTES +
                                    row * (C::PART_COLS * 2) + chunk * 16 + ((col >> 2) & 1) * 8);
      wf[fb][fw][2 * h] = v[0];
      wf[fb][fw][2 * h + 1] = v[1];
    } else {
      const int fa = r - 2 * C::FW;
      const int row = a_row + fa * 32;
      const int chunk = (kk / 8 + a_chk) ^ C::a_swz(row);
      af[fb][fa] = *reinterpret_cast<const u32x4*>(st + row * (BK * 2) + chunk * 16);
    }
  };

  f32x16 acc[C::NACC][C::FW][C::FA];
#pragma unroll
  for (int p = 0; p < C::NACC; ++p)
#pragma unroll
    for (int i = 0; i < C::FW; ++i)
#pragma unroll
      for (int j = 0; j < C::FA; ++j) acc[p][i][j] = f32x16{};

  // One K step on stage ST.  The MFMAs of each sub-step are interleaved with
  // the fragment reads of the next sub-step (first half of the MFMAs) and
  // with half a step of DMA (second half): sub-step 0 finishes step
  // it+STAGES-1, and after the barrier -- once every wave has finished
  // reading stage ST -- the last sub-step starts step it+STAGES into stage ST
  // itself.  Spreading the DMA keeps the address FIFO from backing up into
  // the MFMA stream, and the barrier overlaps the MFMA tail of sub-step 0.
  constexpr int LH = C::LOADS / 2;  // DMA instructions in the first half-step
  auto kstep = [&](int it, auto st_c, auto phase_c) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    constexpr int PH = decltype(phase_c)::value;
    constexpr int NMF = C::FW * C::FA;
    // fragment reads ride on MFMA slots [0, HALF), the DMA on [DBEGIN, NMF);
    // with a single MFMA per sub-step both use slot 0
    constexpr int HALF = NMF / 2 > 0 ? NMF / 2 : 1;
    constexpr int DSLOTS = NMF - HALF > 0 ? NMF - HALF : 1;
    constexpr int DBEGIN = NMF - DSLOTS;
    using Next = std::integral_constant<int, (ST + 1) % STAGES>;
    using Prev = std::integral_constant<int, (ST + STAGES - 1) % STAGES>;
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub) {
      const int fb = sub & 1;
      const bool last = sub == C::NSUB - 1;
      if (last) {
        wait_vmcnt<(STAGES - 2) * C::LOADS>();
        __syncthreads();
      }
      // this sub-step's DMA: [d0, d1) of step dstep into stage DS
      const int nd = (sub == 0) ? C::LOADS - LH : (last ? LH : 0);
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        const int i = q / C::FA, j = q % C::FA;
        acc[PH][i][j] = mfma32(wf[fb][i], af[fb][j], acc[PH][i][j]);
        if (q < HALF) {
#pragma unroll
          for (int x = q * NFRAG / HALF; x < (q + 1) * NFRAG / HALF; ++x) {
            if (last) frag(Next{}, 0, fb ^ 1, x);
            else frag(st_c, sub + 1, fb ^ 1, x);
          }
        }
        if (nd > 0 && q >= DBEGIN) {
#pragma unroll
          for (int x = (q - DBEGIN) * nd / DSLOTS; x < (q - DBEGIN + 1) * nd / DSLOTS; ++x) {
            if (sub == 0) dma(it + STAGES - 1, Prev{}, LH + x);
            else dma(it + STAGES, st_c, x);
          }
        }
        // keep this MFMA and its share of memory work together, in order
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // STAGES K steps, the stage ring unrolled
  auto round = [&](int it0, auto phase_c) __attribute__((always_inline)) {
    [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
      (kstep(it0 + S, std::integral_constant<int, S>{}, phase_c), ...);
    }(std::make_integer_sequence<int, STAGES>{});
  };
  // steps [b, e) with b on a ring boundary: whole rounds, then the remaining
  // steps (fewer than STAGES), each with its compile-time stage
  auto run = [&](int b, int e, auto phase_c) __attribute__((always_inline)) {
    int it = b;
    for (; it + STAGES <= e; it += STAGES) round(it, phase_c);
    [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
      ((it + S < e ? (kstep(it + S, std::integral_constant<int, S>{}, phase_c), 0) : 0), ...);
    }(std::make_integer_sequence<int, STAGES - 1>{});
  };

  // ---- prologue -------------------------------------------------------------------
  // steps 0..STAGES-2 whole and the first half of step STAGES-1, as if the
  // loop had already been running
  auto fill = [&](int it, auto st_c, int q0, int q1) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < C::LOADS; ++q)
      if (q >= q0 && q < q1) dma(it, st_c, q);
  };
  [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
    (fill(S, std::integral_constant<int, S>{}, 0, C::LOADS), ...);
  }(std::make_integer_sequence<int, STAGES - 1>{});
  fill(STAGES - 1, std::integral_constant<int, STAGES - 1>{}, 0, LH);
  wait_vmcnt<(STAGES - 2) * C::LOADS + LH>();
  __syncthreads();
#pragma unroll
  for (int r = 0; r < NFRAG; ++r) frag(std::integral_constant<int, 0>{}, 0, 0, r);

  // ---- main loop ----------------------------------------------------------------
  if constexpr (MODE == MODE_SYNC) {
    run(0, nk0, std::integral_constant<int, 0>{});
    // Gate finished: SiLU on the register-resident Gate accumulator while the
    // next Up weight tiles are still in flight.
#pragma unroll
    for (int i = 0; i < C::FW; ++i)
#pragma unroll
      for (int j = 0; j < C::FA; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[0][i][j][r] = silu(acc[0][i][j][r]);
    run(nk0, total, std::integral_constant<int, 1>{});
  } else {
    run(0, total, std::integral_constant<int, 0>{});
  }

  // ---- epilogue: bf16 tile through LDS, then 16-byte row stores -------------------
  wait_vmcnt<0>();
  __syncthreads();
  const int h32 = lane >> 5;
  if constexpr (MODE == MODE_PAIR) {
    // The Gate waves hand SiLU(Gate) of their rows and columns to the Up
    // waves through LDS in fp32; the Up waves form the products and store Y
    // straight from registers, 4 columns (8 bytes) per lane.
    float* ss = reinterpret_cast<float*>(smem);  // [BM][SLD]
    const bool gate_wave = wn * C::WTW < C::PART_COLS;
    if (gate_wave) {
#pragma unroll
      for (int i = 0; i < C::FW; ++i)
#pragma unroll
        for (int j = 0; j < C::FA; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = a_row + j * 32;
            const int col = wn * C::WTW + i * 32 + 8 * q + 4 * h32;
            const f32x16& d = acc[0][i][j];
            *reinterpret_cast<f32x4*>(ss + row * C::SLD + col) =
                f32x4{silu(d[4 * q]), silu(d[4 * q + 1]), silu(d[4 * q + 2]), silu(d[4 * q + 3])};
          }
    }
    __syncthreads();
    if (!gate_wave) {
#pragma unroll
      for (int i = 0; i < C::FW; ++i)
#pragma unroll
        for (int j = 0; j < C::FA; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = a_row + j * 32;
            const int col = wn * C::WTW - C::PART_COLS + i * 32 + 8 * q + 4 * h32;
            const f32x4 sv = *reinterpret_cast<const f32x4*>(ss + row * C::SLD + col);
            const f32x16& d = acc[0][i][j];
            const int gr = m0 + row, gc = y0 + col;
            if (gr < M && gc < N)  // N % 8 == 0: four columns are in range together
              *reinterpret_cast<u32x2*>(Y + (size_t)gr * ldy + gc) =
                  u32x2{pack_bf16x2(sv[0] * d[4 * q], sv[1] * d[4 * q + 1]),
                        pack_bf16x2(sv[2] * d[4 * q + 2], sv[3] * d[4 * q + 3])};
          }
    }
    return;
  }
  uint16_t* ys = reinterpret_cast<uint16_t*>(smem);  // [BM][YLD]
#pragma unroll
  for (int i = 0; i < C::FW; ++i)
#pragma unroll
    for (int j = 0; j < C::FA; ++j) {
      const int row = a_row + j * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // registers 4q..4q+3 hold weight columns wcl..wcl+3 of this lane's row
        const int wcl = wn * C::WTW + i * 32 + 8 * q + 4 * h32;
        const f32x16& d = acc[0][i][j];
        if constexpr (MODE == MODE_INTERLEAVE) {
          const float ya = silu(d[4 * q + 0]) * d[4 * q + 1];  // pair (wcl, wcl+1)
          const float yb = silu(d[4 * q + 2]) * d[4 * q + 3];  // pair (wcl+2, wcl+3)
          *reinterpret_cast<uint32_t*>(ys + row * C::YLD + wcl / 2) = pack_bf16x2(ya, yb);
        } else {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            y[e] = (MODE == MODE_SYNC) ? d[4 * q + e] * acc[C::NACC - 1][i][j][4 * q + e]
                                       : d[4 * q + e];
          *reinterpret_cast<u32x2*>(ys + row * C::YLD + wcl) =
              u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        }
      }
    }
  __syncthreads();
  constexpr int YCH = C::BNY / 8;
  for (int p = tid; p < BM * YCH; p += C::kThreads) {
    const int row = p / YCH, cq = p % YCH;
    const int gr = m0 + row, gc = y0 + cq * 8;
    if (gr < M && gc < N)
      *reinterpret_cast<u32x4*>(Y + (size_t)gr * ldy + gc) =
          *reinterpret_cast<const u32x4*>(ys + row * C::YLD + cq * 8);
  }
}

template <int MODE, int BM, int BNW, int BK, int STAGES, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void tiled_kernel(const uint16_t* __restrict__ A,
                                                    const uint16_t* __restrict__ W1,
                                                    const uint16_t* __restrict__ W2,
                                                    uint16_t* __restrict__ Y, int M, int N,
                                                    int K, int ldw, int ldy, int group_m) {
  using C = Tiled<MODE, BM, BNW, BK, STAGES, WGM, WGN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];
  // workgroups of one XCD (8 per chip, each with its own L2) take a
  // contiguous range of the tile order
  const int ntm = (M + BM - 1) / BM;
  const int ntn = (N + C::BNY - 1) / C::BNY;
  int tm, tn;
  tile_of(xcd_remap(blockIdx.x, gridDim.x), ntm, ntn, group_m, tm, tn);
  tiled_tile<MODE, BM, BNW, BK, STAGES, WGM, WGN>(A, W1, W2, Y, M, N, K, ldw, ldy, tm * BM, tn,
                                                  smem);
}

// Same tiles, with a split tail: when the tiles do not fill whole rounds of
// workgroups (one per CU), the big tiles of the last, partial round are each
// computed as four quarter tiles (BM/2 x BNW/2) by four workgroups, which
// spreads that round over four times as many CUs.  Workgroups [0, n_big)
// take big tiles 0 .. n_big-1 of the tile order; workgroup n_big + u takes
// quarter u % 4 of big tile n_big + u / 4.  Both tile kinds run on the same
// eight waves (SWGM x SWGN for the quarter tiles).
template <int MODE, int BM, int BNW, int BK, int STAGES, int WGM, int WGN, int SWGM, int SWGN>
__global__ __launch_bounds__(64 * WGM * WGN) void tiled_split_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W2, uint16_t* __restrict__ Y, int M, int N, int K, int ldw,
    int ldy, int group_m, int n_big) {
  using Big = Tiled<MODE, BM, BNW, BK, STAGES, WGM, WGN>;
  using Small = Tiled<MODE, BM / 2, BNW / 2, BK, STAGES, SWGM, SWGN>;
  static_assert(Big::kThreads == Small::kThreads, "one workgroup size for both tile kinds");
  constexpr int LDS = Big::LDS_BYTES > Small::LDS_BYTES ? Big::LDS_BYTES : Small::LDS_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];
  const int ntm = (M + BM - 1) / BM;
  const int ntn = (N + Big::BNY - 1) / Big::BNY;
  int tm, tn;
  if ((int)blockIdx.x < n_big) {
    tile_of(xcd_remap(blockIdx.x, n_big), ntm, ntn, group_m, tm, tn);
    tiled_tile<MODE, BM, BNW, BK, STAGES, WGM, WGN>(A, W1, W2, Y, M, N, K, ldw, ldy, tm * BM,
                                                    tn, smem);
  } else {
    const int u = blockIdx.x - n_big, q = u & 3;
    tile_of(n_big + u / 4, ntm, ntn, group_m, tm, tn);
    const int m0 = tm * BM + (q >> 1) * (BM / 2);
    const int tq = 2 * tn + (q & 1);  // column tile in quarter-tile units
    if (m0 >= M || tq * Small::BNY >= N) return;  // quarter past a ragged edge
    tiled_tile<MODE, BM / 2, BNW / 2, BK, STAGES, SWGM, SWGN>(A, W1, W2, Y, M, N, K, ldw, ldy,
                                                              m0, tq, smem);
  }
}

// ============================================================================
// Persistent LDS-tiled kernel: the next tile's loads under this tile's tail
// ============================================================================
// [RT §Metodologia, Kernel-2, "Sovrapposizione"]: the page overlaps a tile's
// arithmetic with the previous tile's memory traffic.  On MI355X the stores
// are fire-and-forget; what a new tile costs is its pipeline fill, a full
// memory latency before the first MFMA.  Here one workgroup per CU keeps its
// CU for a run of tiles and runs the DMA ring across tile boundaries: K is a
// whole number of rings, so every tile starts on stage 0, and during a tile's
// last STAGES - 1 K steps the ring already loads the first steps of the
// workgroup's next tile (the same DMA slots, with that tile's offsets); the
// next tile's first fragments are read before the epilogue.  The epilogue
// (SiLU, pair multiply, bf16) stages Y through an LDS region of its own beside
// the ring, a slab of wave rows at a time, so the loads in flight are never
// overwritten, and its 16-byte stores overlap the next tile's first steps.
// Tiles follow the XCD-aware launch order: the workgroups of one XCD take that
// XCD's contiguous range of the order in turn.  A last round at most a quarter
// full runs as quarter tiles after the loop, as in tiled_split_kernel.
template <int MODE, int BM, int BNW, int BK, int STAGES, int WGM, int WGN>
struct Persist {
  using C = Tiled<MODE, BM, BNW, BK, STAGES, WGM, WGN>;
  static_assert(MODE == MODE_INTERLEAVE || MODE == MODE_GEMM, "one K loop per tile");
  static_assert(!C::NEED_JUNK, "every wave owns chunks of every K step");
  static constexpr int RING = STAGES * C::STAGE_BYTES;
  static constexpr int LDS_BYTES = 160 * 1024;
  static constexpr int YCH = C::BNY / 8;  // 16-byte chunks per Y row
  static_assert(YCH % 16 == 0, "the staging swizzle permutes aligned groups of 16 chunks");
  static constexpr int WPP = (LDS_BYTES - RING) / (C::BNY * 2) / C::WTM;  // wave rows per slab
  static_assert(WPP >= 1 && WGM % WPP == 0, "Y staging");
  static constexpr int PASSES = WGM / WPP;
  static constexpr int SROWS = WPP * C::WTM;  // Y rows staged per pass
  static_assert(RING + SROWS * C::BNY * 2 <= LDS_BYTES, "LDS");
  // chunk c of staged row r at c ^ y_swz(r): a wave writes one column of 32
  // consecutive rows at a time, which this spreads over 16 chunks
  __host__ __device__ static constexpr int y_swz(int row) { return row & 15; }
};

// Tiles t0, t0 + stride, ... (< t_end) of the launch order, one after another
// on this workgroup, with the ring running across tile boundaries.  K must be
// a positive multiple of BK * STAGES.  Ends with every DMA drained.
//
// Registers: the accumulators of a tile are live through its epilogue, so no
// per-thread address may be: everything per-thread is derived, inside each
// tile's iteration, from a copy of the thread index that the compiler cannot
// see through (an empty asm statement), and only wave-uniform tile offsets
// cross the epilogue.
template <int MODE, int BM, int BNW, int BK, int STAGES, int WGM, int WGN>
__device__ __forceinline__ void tiled_persist(const uint16_t* __restrict__ A,
                                              const uint16_t* __restrict__ W,
                                              uint16_t* __restrict__ Y, int M, int N, int K,
                                              int ldw, int ldy, int group_m, int t0, int stride,
                                              int t_end, uint8_t* smem) {
  using C = Tiled<MODE, BM, BNW, BK, STAGES, WGM, WGN>;
  using P = Persist<MODE, BM, BNW, BK, STAGES, WGM, WGN>;
  static_assert(C::swizzles_permute_rows(), "LDS swizzle is not a permutation of a row");

  const int ntm = (M + BM - 1) / BM, ntn = (N + C::BNY - 1) / C::BNY;
  const int nk = K / BK;  // a multiple of STAGES
  const int wave_u = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave_u / WGN, wn = wave_u % WGN;
  const int wcols = (MODE == MODE_INTERLEAVE) ? 2 * N : N;
  const uint32_t wbytes = (uint32_t)(((size_t)(K - 1) * ldw + wcols) * 2);
  const i32x4 rsA = make_rsrc(A, (uint32_t)((size_t)M * K * 2));
  const i32x4 rsW = make_rsrc(W, wbytes);
  const uint32_t lds0 = lds_addr(smem);
  uint16_t* ys = reinterpret_cast<uint16_t*>(smem + P::RING);  // [SROWS][BNY], swizzled

  // A tile's offsets are wave-uniform (scalar registers).  K is a multiple of
  // BK, so no chunk reaches past K; rows of A past M lie past the end of A and
  // read zeros by the buffer bound, so only weight columns past the matrix
  // need a mask.  A tile at or past t_end gets offsets out of range everywhere.
  struct TileOffs {
    uint32_t a;  // byte offset of the tile's first row of A
    uint32_t w;  // byte offset of its first weight column
    int wlim;    // weight columns of the tile inside the matrix
  };
  auto offsets = [&](int t) __attribute__((always_inline)) {
    TileOffs o{(uint32_t)M * (uint32_t)K * 2u, 0u, 0};
    if (t < t_end) {
      int tm, tn;
      tile_of(t, ntm, ntn, group_m, tm, tn);
      o.a = (uint32_t)(tm * BM) * (uint32_t)K * 2u;
      o.w = (uint32_t)(tn * BNW) * 2u;
      o.wlim = wcols - tn * BNW;
    }
    o.a = __builtin_amdgcn_readfirstlane(o.a);
    o.w = __builtin_amdgcn_readfirstlane(o.w);
    o.wlim = __builtin_amdgcn_readfirstlane(o.wlim);
    return o;
  };
  // this tile's offsets and the next tile's
  TileOffs oc = offsets(t0), on = oc;
  u32x4 wf[2][C::FW], af[2][C::FA];  // fragments (double-buffered by sub-step)

  for (int t = t0; t < t_end; t += stride) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;

    // per-thread DMA parts (the tile's parts are in oc / on)
    uint32_t a_base[C::A_LOADS], w_base[C::W_LOADS];
    int w_c8[C::W_LOADS];
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      const int p = tid + C::kThreads * i;
      const int row = p / C::ACH;
      const int c = (p % C::ACH) ^ C::a_swz(row);
      a_base[i] = (uint32_t)(row * K + c * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < C::W_LOADS; ++i) {
      const int p = tid + C::kThreads * i;
      const int row = p / C::WCH;
      const int c = (p % C::WCH) ^ C::w_swz(row);
      w_base[i] = (uint32_t)(row * ldw + c * 8) * 2u;
      w_c8[i] = c * 8;
    }
    // DMA instruction q of K step `it` into stage ST: steps [0, nk) of the
    // current tile, steps [nk, nk + STAGES) the first ones of the next tile
    auto dma = [&](int it, auto st_c, int q) __attribute__((always_inline)) {
      constexpr int ST = decltype(st_c)::value;
      const bool nxt = it >= nk;  // wave-uniform
      const TileOffs o = nxt ? on : oc;
      const uint32_t k0 = (uint32_t)((nxt ? it - nk : it) * BK);
      const uint32_t sbase = lds0 + ST * C::STAGE_BYTES;
      if (q < C::A_LOADS) {
        const int p0 = C::kThreads * q + 64 * wave_u;
        lds_dma16(sbase + p0 * 16, a_base[q] + o.a + k0 * 2u, rsA);
      } else {
        const int i = q - C::A_LOADS;
        const int p0 = C::kThreads * i + 64 * wave_u;
        const uint32_t off =
            w_c8[i] < o.wlim ? w_base[i] + o.w + k0 * (uint32_t)ldw * 2u : kOutOfRange;
        lds_dma16(sbase + C::A_BYTES + p0 * 16, off, rsW);
      }
    };

    // fragments (as in tiled_tile)
    const int g16 = lane >> 4, s16 = lane & 15;
    const int w_row = 8 * (g16 >> 1) + (s16 >> 2);
    const int w_col = wn * C::WTW + 16 * (g16 & 1) + 4 * (s16 & 3);
    const int a_row = wm * C::WTM + (lane & 31);
    const int a_chk = lane >> 5;
    constexpr int NFRAG = 2 * C::FW + C::FA;
    auto frag = [&](auto st_c, int sub, int fb, int r) __attribute__((always_inline)) {
      constexpr int ST = decltype(st_c)::value;
      const uint8_t* st = smem + ST * C::STAGE_BYTES;
      const int kk = sub * 16;
      if (r < 2 * C::FW) {
        const int fw = r >> 1, h = r & 1;
        const int col = w_col + fw * 32;
        const int row = kk + w_row + 4 * h;
        const int chunk = (col >> 3) ^ C::w_swz(row);
        const u32x2 v = lds_read_tr16(st + C::A_BYTES + row * (BNW * 2) + chunk * 16 +
                                      ((col >> 2) & 1) * 8);
        wf[fb][fw][2 * h] = v[0];
        wf[fb][fw][2 * h + 1] = v[1];
      } else {
        const int fa = r - 2 * C::FW;
        const int row = a_row + fa * 32;
        const int chunk = (kk / 8 + a_chk) ^ C::a_swz(row);
        af[fb][fa] = *reinterpret_cast<const u32x4*>(st + row * (BK * 2) + chunk * 16);
      }
    };

    f32x16 acc[C::FW][C::FA];

    // one K step on stage ST (the schedule of tiled_tile); the tile's last
    // step reads the next tile's first fragments, whose data has landed by
    // then (its wait and barrier cover step nk, the next tile's step 0)
    constexpr int LH = C::LOADS / 2;
    auto kstep = [&](int it, auto st_c) __attribute__((always_inline)) {
      constexpr int ST = decltype(st_c)::value;
      constexpr int NMF = C::FW * C::FA;
      constexpr int HALF = NMF / 2 > 0 ? NMF / 2 : 1;
      constexpr int DSLOTS = NMF - HALF > 0 ? NMF - HALF : 1;
      constexpr int DBEGIN = NMF - DSLOTS;
      using Next = std::integral_constant<int, (ST + 1) % STAGES>;
      using Prev = std::integral_constant<int, (ST + STAGES - 1) % STAGES>;
#pragma unroll
      for (int sub = 0; sub < C::NSUB; ++sub) {
        const int fb = sub & 1;
        const bool last = sub == C::NSUB - 1;
        if (last) {
          wait_vmcnt<(STAGES - 2) * C::LOADS>();
          __syncthreads();
        }
        const int nd = (sub == 0) ? C::LOADS - LH : (last ? LH : 0);
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
          const int i = q / C::FA, j = q % C::FA;
          acc[i][j] = mfma32(wf[fb][i], af[fb][j], acc[i][j]);
          if (q < HALF) {
#pragma unroll
            for (int x = q * NFRAG / HALF; x < (q + 1) * NFRAG / HALF; ++x) {
              if (last) frag(Next{}, 0, fb ^ 1, x);
              else frag(st_c, sub + 1, fb ^ 1, x);
            }
          }
          if (nd > 0 && q >= DBEGIN) {
#pragma unroll
            for (int x = (q - DBEGIN) * nd / DSLOTS; x < (q - DBEGIN + 1) * nd / DSLOTS; ++x) {
              if (sub == 0) dma(it + STAGES - 1, Prev{}, LH + x);
              else dma(it + STAGES, st_c, x);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    auto round = [&](int it0) __attribute__((always_inline)) {
      [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
        (kstep(it0 + S, std::integral_constant<int, S>{}), ...);
      }(std::make_integer_sequence<int, STAGES>{});
    };

    if (t == t0) {
      // prologue: the first tile's steps 0..STAGES-2 and half of STAGES-1
      auto fill = [&](int it, auto st_c, int q0, int q1) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < C::LOADS; ++q)
          if (q >= q0 && q < q1) dma(it, st_c, q);
      };
      [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
        (fill(S, std::integral_constant<int, S>{}, 0, C::LOADS), ...);
      }(std::make_integer_sequence<int, STAGES - 1>{});
      fill(STAGES - 1, std::integral_constant<int, STAGES - 1>{}, 0, LH);
      wait_vmcnt<(STAGES - 2) * C::LOADS + LH>();
      __syncthreads();
#pragma unroll
      for (int r = 0; r < NFRAG; ++r) frag(std::integral_constant<int, 0>{}, 0, 0, r);
    }
    // this tile's step-0 fragments are in registers (read above, or in the
    // previous tile's last step)
#pragma unroll
    for (int i = 0; i < C::FW; ++i)
#pragma unroll
      for (int j = 0; j < C::FA; ++j) acc[i][j] = f32x16{};
    on = offsets(t + stride);
    for (int it = 0; it < nk; it += STAGES) round(it);
    // The next tile's first STAGES - 1 steps (and half of the one after) are
    // in flight or landed, and its step-0 fragments are in registers.

    // ---- epilogue: one slab of wave rows at a time through the staging region
    const int h32 = lane >> 5;
    int tm, tn;
    tile_of(t, ntm, ntn, group_m, tm, tn);
    const int m0 = tm * BM, y0 = tn * C::BNY;
#pragma unroll
    for (int pass = 0; pass < P::PASSES; ++pass) {
      if (wm / P::WPP == pass) {
#pragma unroll
        for (int i = 0; i < C::FW; ++i)
#pragma unroll
          for (int j = 0; j < C::FA; ++j) {
            const int row = (wm % P::WPP) * C::WTM + (lane & 31) + j * 32;  // staged row
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int wcl = wn * C::WTW + i * 32 + 8 * q + 4 * h32;
              const f32x16& d = acc[i][j];
              if constexpr (MODE == MODE_INTERLEAVE) {
                const int col = wcl / 2;
                const int e = (((col >> 3) ^ P::y_swz(row)) << 3) | (col & 7);
                const float ya = silu(d[4 * q + 0]) * d[4 * q + 1];  // pair (wcl, wcl+1)
                const float yb = silu(d[4 * q + 2]) * d[4 * q + 3];  // pair (wcl+2, wcl+3)
                *reinterpret_cast<uint32_t*>(ys + row * C::BNY + e) = pack_bf16x2(ya, yb);
              } else {
                const int e = (((wcl >> 3) ^ P::y_swz(row)) << 3) | (wcl & 7);
                *reinterpret_cast<u32x2*>(ys + row * C::BNY + e) =
                    u32x2{pack_bf16x2(d[4 * q], d[4 * q + 1]),
                          pack_bf16x2(d[4 * q + 2], d[4 * q + 3])};
              }
            }
          }
      }
      __syncthreads();
      for (int p = tid; p < P::SROWS * P::YCH; p += C::kThreads) {
        const int row = p / P::YCH, cq = p % P::YCH;
        const int gr = m0 + pass * P::SROWS + row, gc = y0 + cq * 8;
        if (gr < M && gc < N)
          *reinterpret_cast<u32x4*>(Y + (size_t)gr * ldy + gc) = *reinterpret_cast<const u32x4*>(
              ys + row * C::BNY + ((cq ^ P::y_swz(row)) << 3));
      }
      // the next pass (or the next tile's epilogue, after its K loop's
      // barriers) overwrites the staging rows
      if (pass + 1 < P::PASSES) __syncthreads();
    }
    oc = on;
  }
  // the zero loads issued past the last tile still write LDS
  wait_vmcnt<0>();
  __syncthreads();
}

template <int MODE, int BM, int BNW, int BK, int STAGES, int WGM, int WGN, int SWGM, int SWGN>
__global__ __launch_bounds__(64 * WGM * WGN) void tiled_persist_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, uint16_t* __restrict__ Y,
    int M, int N, int K, int ldw, int ldy, int group_m, int n_big, int n_quarter) {
  using P = Persist<MODE, BM, BNW, BK, STAGES, WGM, WGN>;
  using Small = Tiled<MODE, BM / 2, BNW / 2, BK, STAGES, SWGM, SWGN>;
  static_assert(Small::kThreads == P::C::kThreads, "one workgroup size for both tile kinds");
  static_assert(Small::LDS_BYTES <= P::LDS_BYTES, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[P::LDS_BYTES];
  // workgroup b runs on XCD b % 8; each XCD owns a contiguous range of the
  // first n_big tiles of the order, which its workgroups take in turn
  const int G = gridDim.x, b = blockIdx.x;
  const int x = b % 8, i = b / 8;
  const int gx = G / 8 + (x < G % 8 ? 1 : 0);
  const int q = n_big / 8, r = n_big % 8;
  const int lo = x * q + min(x, r), cnt = q + (x < r ? 1 : 0);
  if (i < cnt)
    tiled_persist<MODE, BM, BNW, BK, STAGES, WGM, WGN>(A, W, Y, M, N, K, ldw, ldy, group_m,
                                                       lo + i, gx, lo + cnt, smem);
  // the short last round, as quarter tiles (BM/2 x BNW/2): quarter u % 4 of
  // big tile n_big + u / 4
  const int ntm = (M + BM - 1) / BM, ntn = (N + P::C::BNY - 1) / P::C::BNY;
  for (int u = b; u < n_quarter; u += G) {
    int tm, tn;
    tile_of(n_big + u / 4, ntm, ntn, group_m, tm, tn);
    const int m0 = tm * BM + ((u & 3) >> 1) * (BM / 2);
    const int tq = 2 * tn + (u & 1);
    if (m0 < M && tq * Small::BNY < N)
      tiled_tile<MODE, BM / 2, BNW / 2, BK, STAGES, SWGM, SWGN>(A, W, W, Y, M, N, K, ldw, ldy,
                                                                m0, tq, smem);
    __syncthreads();  // the next quarter tile's loads overwrite this one's LDS
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
      // MT == 1 is chosen for M <= 16: one row group, each weight read once
      u32x2 g = ok ? (MT == 1 ? load8_stream(p1 + (size_t)r * N) : load8(p1 + (size_t)r * N))
                   : u32x2{0, 0};
      u32x2 u = ok ? (MT == 1 ? load8_stream(p2 + (size_t)r * N) : load8(p2 + (size_t)r * N))
                   : u32x2{0, 0};
      rows[r] = u32x4{g[0], g[1], u[0], u[1]};
    }
  } else {
    const int ld = (MODE == MODE_INTERLEAVE) ? 2 * N : N;
    const int c = slab * 128 + cg * 8;
    const bool ok = kin && c < ld;
    const uint16_t* p = W1 + (size_t)k * ld + c;
#pragma unroll
    for (int r = 0; r < 8; ++r)
      rows[r] = ok ? (MT == 1 ? load16_stream(p + (size_t)r * ld) : load16(p + (size_t)r * ld))
                   : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + mt * 16 + (lane & 15);
    af[mt] = (kin && m < M) ? load16(A + (size_t)m * K + k) : u32x4{0, 0, 0, 0};
  }
}

template <int MODE, int MT, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(MT == 1 ? 4 : 2)))
void skinny_kernel(const uint16_t* __restrict__ A,
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

  // One register set per wave: while a wave transposes and multiplies, the
  // other waves of the SIMD (four per SIMD at MT = 1) have their loads in
  // flight, which keeps more bytes outstanding per CU than a per-wave double
  // buffer that would cost the occupancy.
  for (int s = s_begin; s < s_end; ++s) {
    u32x4 rows[8], af[MT];
    skinny_load<MODE, MT>(A, W1, W2, M, N, K, m0, slab, lane, s, rows, af);
    mma(rows, af);
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
// Fragment-ordered weights: split-K streaming without transposition
// ============================================================================
// W_fused [K, 2N] ([RT §Metodologia, Kernel-2]) stored once, offline, in the
// order the 16x16x32 MFMA consumes it.  The columns are cut into slabs of 128
// and K into steps of 32; block (slab s, step t) is 4096 values (8 KB):
//   P[((s T + t) 8 + c) 512 + (16 g + l) 8 + e] = W_fused[32 t + 8 g + e][128 s + 8 l + c]
// with T = ceil(K / 32), c, e < 8, g < 4, l < 16, and zeros outside [K, 2N].
// The 1 KB run c of a block is the B fragment of MFMA c for all 64 lanes (lane
// 16 g + l: 8 consecutive k of column 128 s + 8 l + c), so every load
// instruction reads 1 KB contiguous, a block is 8 KB contiguous, and the
// blocks of a slab follow one another.  The accumulators of MFMA 2q and 2q+1
// hold the Gate and the Up column of output 64 s + 4 l + q in the same lane,
// as in the skinny kernel.
//
// A workgroup takes CH of the 8 MFMA column groups of one slab (CH = 8, 4 or
// 2; CH/2 outputs per lane and row), i.e. a contiguous CH KB run of every
// block of the slab (with CH = 8 the whole slab, one contiguous span).  Each
// CU streams at a bounded rate, so the time follows the most loaded CU:
// splitting a slab into 8/CH workgroups evens the load (Qwen2.5-7B decode:
// 296 slabs on 256 CUs, run as 592 half slabs).
//
// Waves of a workgroup take the slab's steps in turn (wave w: t = w, w + NW,
// ...), so at any time they read neighbouring blocks; each wave keeps two
// steps of loads in flight (two register sets, the load of the step after
// next issued as soon as a set's MFMAs are issued).  The fp32 partials are
// reduced through LDS in wave order before SiLU, as in skinny_kernel.
template <int MT, int NW, int CH>
struct Packed {
  static_assert(CH == 2 || CH == 4 || CH == 8, "column groups per workgroup");
  static constexpr int kThreads = 64 * NW;
  static constexpr int LDS_BYTES = NW * MT * CH * 64 * 16;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static constexpr int PARTS = 8 / CH;     // workgroups per slab
  static constexpr int COLS_Y = 8 * CH;    // output columns per workgroup
};

template <int MT, int CH>
__device__ __forceinline__ void packed_load(const uint16_t* __restrict__ A,
                                            const uint16_t* __restrict__ wp, int M, int K,
                                            int m0, int lane, int step, u32x4 (&b)[CH],
                                            u32x4 (&af)[MT]) {
  // Activations first.  Every lane loads, so no branch skips a load and the
  // in-order load counter stays exact: rows past M re-read row M-1 (an output
  // row depends only on its own A row, and those rows are never stored), k
  // past K re-reads the last octet and is zeroed by the caller right before
  // its MFMAs (M >= 1 and K >= 8 here).
  const int k = min(step * 32 + (lane >> 4) * 8, K - 8);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(m0 + mt * 16 + (lane & 15), M - 1);
    af[mt] = load16(A + (size_t)m * K + k);
  }
  const uint16_t* p = wp + (size_t)step * 4096;
#pragma unroll
  for (int c = 0; c < CH; ++c) b[c] = MT == 1 ? load16_stream(p + c * 512) : load16(p + c * 512);
}

// Part `part` (CH of the 8 column groups) of slab `slab`, rows m0 ... m0 +
// 16 MT - 1, by the workgroup's NW waves; red: LDS for the wave reduction
// (NW MT CH 64 f32x4).
template <int MT, int NW, int CH>
__device__ __forceinline__ void packed_unit(const uint16_t* __restrict__ A,
                                            const uint16_t* __restrict__ P,
                                            uint16_t* __restrict__ Y, int M, int N, int K,
                                            int slab, int part, int m0, f32x4* red) {
  using C = Packed<MT, NW, CH>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nsteps = (K + 31) / 32;
  // this lane's 16 bytes in each of the workgroup's 1 KB runs (column groups
  // part*CH ... part*CH + CH-1) of the slab's blocks
  const uint16_t* wp = P + (size_t)slab * (size_t)nsteps * 4096 + part * CH * 512 + lane * 8;

  f32x4 acc[MT][CH];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[mt][c] = f32x4{};

  // MFMAs of one step; k of this lane's octet past K contributes zero
  auto mma = [&](const u32x4 (&b)[CH], const u32x4 (&af)[MT], int step) {
    const bool kin = step * 32 + (lane >> 4) * 8 < K;  // K % 8 == 0
    u32x4 a[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a[mt] = kin ? af[mt] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt][c] = mfma16(a[mt], b[c], acc[mt][c]);
  };

  // this wave's steps: wave, wave + NW, ...
  if constexpr (MT == 1) {
    // two steps are loaded together and then multiplied, then an odd last
    // one.  With one row group the loads of a pair already cover the memory
    // latency; the software-pipelined form below measured 6 % slower here
    // (7B decode shape: 45.7 vs 48.7 us, one box), as did fencing the loads
    // and MFMAs apart with scheduling barriers (47.6 us).
    u32x4 b0[CH], a0[MT], b1[CH], a1[MT];
    int s = wave;
    for (; s + NW < nsteps; s += 2 * NW) {
      packed_load<MT, CH>(A, wp, M, K, m0, lane, s, b0, a0);
      packed_load<MT, CH>(A, wp, M, K, m0, lane, s + NW, b1, a1);
      mma(b0, a0, s);
      mma(b1, a1, s + NW);
    }
    if (s < nsteps) {
      packed_load<MT, CH>(A, wp, M, K, m0, lane, s, b0, a0);
      mma(b0, a0, s);
    }
  } else if (wave < nsteps) {
    // several row groups: n steps software-pipelined, taken in pairs with
    // both MFMA groups unconditional, then an odd one; a load past the last
    // step re-reads it (in bounds, unused).  The scheduling barriers keep
    // each set's loads issued before the MFMAs that wait for the other set,
    // so two steps stay in flight.
    const int n = (nsteps - 1 - wave) / NW + 1;
    const int last = wave + (n - 1) * NW;
    u32x4 b0[CH], a0[MT], b1[CH], a1[MT];
    packed_load<MT, CH>(A, wp, M, K, m0, lane, wave, b0, a0);
    int s = wave;
    for (int i = 0; i < n / 2; ++i, s += 2 * NW) {
      packed_load<MT, CH>(A, wp, M, K, m0, lane, s + NW, b1, a1);
      __builtin_amdgcn_sched_barrier(0);
      mma(b0, a0, s);
      packed_load<MT, CH>(A, wp, M, K, m0, lane, min(s + 2 * NW, last), b0, a0);
      __builtin_amdgcn_sched_barrier(0);
      mma(b1, a1, s + NW);
    }
    if (n & 1) mma(b0, a0, last);  // b0 holds the last step
  }

  // ---- split-K reduction through LDS (fixed order: wave 0, 1, ..., NW-1) ----
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int c = 0; c < CH; ++c) red[((wave * MT + mt) * CH + c) * 64 + lane] = acc[mt][c];
  __syncthreads();

  // lane l holds W_fused columns 128 slab + 8 l + part*CH + c: the pair
  // (c, c+1), c even, is output column 64 slab + 4 l + (part*CH + c) / 2
  const int col = slab * 64 + (lane & 15) * 4 + part * CH / 2;
  const int rq = (lane >> 4) * 4;
  for (int mt = wave; mt < MT; mt += NW) {
    f32x4 v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      v[c] = red[(mt * CH + c) * 64 + lane];
      for (int w = 1; w < NW; ++w) v[c] += red[((w * MT + mt) * CH + c) * 64 + lane];
    }
    if (col >= N) continue;  // N % 8 == 0: a lane's outputs are all in or all out
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + mt * 16 + rq + r;
      if (row >= M) continue;
      float y[CH / 2];
#pragma unroll
      for (int q = 0; q < CH / 2; ++q) y[q] = silu(v[2 * q][r]) * v[2 * q + 1][r];
      uint16_t* out = Y + (size_t)row * N + col;
      if constexpr (CH == 8) {
        *reinterpret_cast<u32x2*>(out) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      } else if constexpr (CH == 4) {
        *reinterpret_cast<uint32_t*>(out) = pack_bf16x2(y[0], y[1]);
      } else {
        *out = bf16_bits(y[0]);
      }
    }
  }
}

template <int MT, int NW, int CH>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(MT == 1 ? 4 : 2)))
void packed_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ P,
                   uint16_t* __restrict__ Y, int M, int N, int K) {
  using C = Packed<MT, NW, CH>;
  __shared__ __attribute__((aligned(16))) f32x4 red[NW * MT * CH * 64];
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  packed_unit<MT, NW, CH>(A, P, Y, M, N, K, unit / C::PARTS, unit % C::PARTS,
                          (int)blockIdx.y * MT * 16, red);
}

// ---- the same streaming with whole and quarter slabs in one launch ----------
// For slab counts a little above a whole number per CU (Qwen2.5-7B decode:
// 296 slabs on 256 CUs), one size of work unit leaves some CUs a third more
// to stream than others.  Here the first nwhole = floor(slabs / CUs) * CUs
// slabs run as whole slabs, one workgroup of NW waves each, and the rest as
// quarter slabs, so that no CU streams more than one whole and one quarter
// slab beyond an even share.  One row group of 16 rows per grid row.
template <int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(4)))
void packed_mixed_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ P,
                         uint16_t* __restrict__ Y, int M, int N, int K, int nwhole) {
  __shared__ __attribute__((aligned(16))) f32x4 red[NW * 8 * 64];
  const int b = blockIdx.x;
  const int m0 = (int)blockIdx.y * 16;
  if (b < nwhole) {
    packed_unit<1, NW, 8>(A, P, Y, M, N, K, b, 0, m0, red);
  } else {
    const int u = b - nwhole;
    packed_unit<1, NW, 2>(A, P, Y, M, N, K, nwhole + u / 4, u % 4, m0, red);
  }
}

// ---- the same streaming with K split over workgroups (M <= 16) -------------
// When the slabs cannot spread over the CUs (few output columns, e.g. one
// GPU's share of a tensor-parallel MLP at decode), S workgroups share each
// (slab, part): workgroup kp of S takes the contiguous K steps
// [kp n / S, (kp + 1) n / S) of it (n = ceil(K / 32)), reduces its waves in
// LDS, and writes the fp32 partial sums of its 16 x 8CH block to the
// workspace (device-coherent stores).  The last of the S to arrive (a counter per (slab, part)) adds
// the S partials in K order -- fixed, so the result does not depend on which
// arrives last -- and does SiLU and the pair product: every partial is fp32
// and fully reduced before SiLU, as the page requires for split sums across
// tiles ([RT §Risultati], the FP32 cross-tile accumulation behind its 0 %
// error claim).  Nothing waits on another workgroup, so no order of
// execution can stall the launch.  The last one also puts the counter back to
// zero, so a workspace that starts zeroed stays ready for the next call.
//
// Workspace (splitk_workspace_bytes): the counters, then the partials, each
// workgroup's CH KB (CH f32x4 per lane) at its unit index.
template <int NW, int CH>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(4)))
void packed_splitk_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ P,
                          uint16_t* __restrict__ Y, int M, int N, int K, int S,
                          uint32_t* __restrict__ counters, f32x4* __restrict__ partials) {
  using C = Packed<1, NW, CH>;
  __shared__ __attribute__((aligned(16))) f32x4 red[NW * CH * 64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // units in memory order: (slab, part) major, the S pieces of K minor, so
  // concurrently running workgroups stream neighbouring weight runs
  const int unit = blockIdx.x;
  const int sp = unit / S, kp = unit % S;
  const int slab = sp / C::PARTS, part = sp % C::PARTS;
  const int nsteps = (K + 31) / 32;
  const int s0 = (int)((long long)kp * nsteps / S), s1 = (int)((long long)(kp + 1) * nsteps / S);
  const uint16_t* wp = P + (size_t)slab * (size_t)nsteps * 4096 + part * CH * 512 + lane * 8;

  f32x4 acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = f32x4{};
  auto mma = [&](const u32x4 (&b)[CH], const u32x4 (&af)[1], int step) {
    const bool kin = step * 32 + (lane >> 4) * 8 < K;  // K % 8 == 0
    const u32x4 a = kin ? af[0] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = mfma16(a, b[c], acc[c]);
  };
  // this wave's steps s0 + wave, s0 + wave + NW, ... (< s1): pairs loaded
  // together, then multiplied (the one-row-group loop of packed_kernel)
  {
    u32x4 b0[CH], a0[1], b1[CH], a1[1];
    int s = s0 + wave;
    for (; s + NW < s1; s += 2 * NW) {
      packed_load<1, CH>(A, wp, M, K, 0, lane, s, b0, a0);
      packed_load<1, CH>(A, wp, M, K, 0, lane, s + NW, b1, a1);
      mma(b0, a0, s);
      mma(b1, a1, s + NW);
    }
    if (s < s1) {
      packed_load<1, CH>(A, wp, M, K, 0, lane, s, b0, a0);
      mma(b0, a0, s);
    }
  }

  // the waves' sums in LDS, added in wave order by wave 0
#pragma unroll
  for (int c = 0; c < CH; ++c) red[(wave * CH + c) * 64 + lane] = acc[c];
  __syncthreads();
  if (wave != 0) return;
  f32x4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    v[c] = red[c * 64 + lane];
    for (int w = 1; w < NW; ++w) v[c] += red[(w * CH + c) * 64 + lane];
  }

  if (S > 1) {
    // hand the partial over; the last of the S workgroups of this (slab, part)
    // continues with the sum of all S in K order
    f32x4* mine = partials + (size_t)unit * CH * 64;
#pragma unroll
    for (int c = 0; c < CH; ++c) store_agent(mine + c * 64 + lane, v[c]);
    wait_vmcnt<0>();  // the partial has reached the device-coherent level
    uint32_t before = 0;
    if (lane == 0) before = atomic_add_agent(counters + sp, 1u);
    before = (uint32_t)__builtin_amdgcn_readfirstlane((int)before);
    if (before != (uint32_t)(S - 1)) return;
    const f32x4* all = partials + (size_t)sp * S * CH * 64;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      v[c] = load_agent(all + c * 64 + lane);
      for (int k = 1; k < S; ++k) v[c] += load_agent(all + (k * CH + c) * 64 + lane);
    }
    if (lane == 0) counters[sp] = 0u;  // every workgroup of this (slab, part) has counted
  }

  // lane l holds W_fused columns 128 slab + 8 (l % 16) + part CH + c of rows
  // 4 (l / 16) + r: the pair (c, c + 1), c even, is output column
  // 64 slab + 4 (l % 16) + (part CH + c) / 2
  const int col = slab * 64 + (lane & 15) * 4 + part * CH / 2;
  if (col >= N) return;  // N % 8 == 0: a lane's outputs are all in or all out
  const int rq = (lane >> 4) * 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = rq + r;
    if (row >= M) continue;
    float y[CH / 2];
#pragma unroll
    for (int q = 0; q < CH / 2; ++q) y[q] = silu(v[2 * q][r]) * v[2 * q + 1][r];
    uint16_t* out = Y + (size_t)row * N + col;
    if constexpr (CH == 8) {
      *reinterpret_cast<u32x2*>(out) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    } else if constexpr (CH == 4) {
      *reinterpret_cast<uint32_t*>(out) = pack_bf16x2(y[0], y[1]);
    } else {
      *out = bf16_bits(y[0]);
    }
  }
}

// ============================================================================
// FP8 (OCP E4M3) inputs: LDS-tiled interleave and sync kernels
// ============================================================================
// A8 [M, K] and W8 [2N, K] hold E4M3 codes with k contiguous in both; row 2n
// of W8 is Gate column n and row 2n+1 Up column n (the Kernel-2 pairing of
// [RT §Metodologia], each W_fused column stored as a row).  A stored code q
// stands for scale * q with one fp32 scale per tensor; the kernel multiplies
// the finished fp32 accumulators by s_a s_w1 (Gate) and s_a s_w2 (Up) before
// SiLU, so the MFMAs run with unit block scales.
//
// Same skeleton as tiled_kernel: eight (or four) waves, direct HBM -> LDS
// DMA STAGES-1 steps ahead, one barrier per K step, XCD-aware tile order.
// What differs: K steps of 64 (one v_mfma_scale_f32_32x32x64_f8f6f4 per
// 32 x 32 block and step, twice the bf16 rate per cycle) and both tiles are
// k-contiguous rows of 64 bytes with one swizzle and one fragment read: lane
// l takes row l%32 and the 16-byte chunks l/32 and 2 + l/32 of the step, for
// the activation and for the weight source alike (the MFMA only needs the
// two sources to place k the same way).  Per step a wave issues its MFMAs
// weight block by weight block; a weight fragment is re-read for the next
// step as soon as its last MFMA is issued, and the activation fragments are
// double-buffered by step parity (the stage ring has an even length, so the
// parity is a compile-time constant of the unrolled ring).
//
// The sync mode ([RT §Metodologia, Kernel-1]) reads the same W8: its tile
// holds BNW output columns, the Gate phase streams W8 rows 2n (W1 columns)
// and the Up phase rows 2n+1, each over the whole K; between the phases the
// Gate accumulators are scaled and passed through SiLU in registers while
// the first Up tiles are already in flight (the stage ring runs on across
// the phase boundary).
//
// The MX mode is the interleave pairing on MXFP8 inputs: every 32 consecutive
// k of a row of A8 or W8 share one E8M0 scale byte (SA [M, ks], SW [2N, ks]).
// The MFMA applies them itself (per lane, the scale of its row and of the k
// block its fragment half belongs to), so the accumulators come out fully
// scaled.  A 16-byte chunk of a scale row covers 8 K steps; the tile's chunks
// (BM + BNW rows) are loaded by the same DMA into a two-slot ring in LDS, with
// the K step that starts a group of 8 and by that step only: the K loop is
// unrolled by groups of 8 in this mode, so the number of loads a step has in
// flight is still a compile-time constant at every position.  (An extra,
// empty load in each of the other 7 steps cost about a tenth of the MX
// tile's time.)  Each lane reads its scale bytes for the next step with the
// fragments.
template <int MODE, int BM, int BNW, int STAGES, int WGM, int WGN>
struct F8Tiled {
  static constexpr int kWaves = WGM * WGN;
  static_assert(kWaves == 4 || kWaves == 8, "four waves (one per SIMD) or eight (two per SIMD)");
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BK = 64;          // k per step = bytes per tile row
  static constexpr bool SYNC = MODE == MODE_SYNC || MODE == MODE_MX_SYNC;
  static constexpr int BNY = SYNC ? BNW : BNW / 2;  // output columns
  static constexpr int NACC = SYNC ? 2 : 1;         // accumulator sets
  static constexpr int WTM = BM / WGM;   // A rows per wave
  static constexpr int WTW = BNW / WGN;  // W8 rows per wave (per phase in sync mode)
  static constexpr int FA = WTM / 32;
  static constexpr int FW = WTW / 32;
  static_assert(FA >= 1 && FW >= 1 && WTM % 32 == 0 && WTW % 32 == 0, "wave tile");
  static constexpr int A_BYTES = BM * BK;
  static constexpr int W_BYTES = BNW * BK;
  static constexpr int STAGE_BYTES = A_BYTES + W_BYTES;
  static constexpr int A_CHUNKS = BM * 4, W_CHUNKS = BNW * 4;  // 16-byte chunks
  static_assert(A_CHUNKS % 64 == 0 && W_CHUNKS % 64 == 0, "whole waves of chunks");
  static constexpr int A_LOADS = (A_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int W_LOADS = (W_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int LOADS = A_LOADS + W_LOADS;
  static constexpr bool MX = MODE == MODE_MX || MODE == MODE_MX_SYNC;
  static constexpr int SC_CHUNKS = MX ? BM + BNW : 0;  // one 16-byte scale chunk per row
  static constexpr int SC_LOADS = MX ? (SC_CHUNKS + kThreads - 1) / kThreads : 0;
  static_assert(!MX || (BM % 64 == 0 && BNW % 64 == 0), "a wave's scale chunks share one tensor");
  static constexpr int TLOADS = LOADS + SC_LOADS;  // most DMA instructions per thread and K step
  static_assert(STAGES >= 2 && STAGES % 2 == 0, "an even stage ring");
  static_assert((STAGES - 1) * TLOADS <= 63, "vmcnt range");
  // K steps unrolled together: one stage ring, or in MX mode one group of 8
  // steps (the steps one 16-byte scale chunk covers), so that a step's
  // position in its group is a compile-time constant
  static constexpr int UNR = MX ? 8 : STAGES;
  static_assert(UNR % STAGES == 0, "whole stage rings per unrolled block");
  // DMA instructions per thread of the step at position t of the block: the
  // scale chunks travel with the first step of their group only
  __host__ __device__ static constexpr int step_loads(int t) {
    return LOADS + ((MX && t % UNR == 0) ? SC_LOADS : 0);
  }
  // loads a thread may still have in flight at the top of the step at
  // position t, when the step after it must have landed: those of steps
  // t + 2 ... t + STAGES - 1 (the DMA runs STAGES - 1 steps ahead)
  __host__ __device__ static constexpr int in_flight(int t) {
    int n = 0;
    for (int d = 2; d < STAGES; ++d) n += step_loads(t + d);
    return n;
  }
  // the same after the prologue, when step 0 must have landed
  __host__ __device__ static constexpr int prologue_in_flight() {
    int n = 0;
    for (int d = 1; d < STAGES; ++d) n += step_loads(d);
    return n;
  }
  static constexpr int YLD = BNY + 8;
  static constexpr int Y_BYTES = BM * YLD * 2;
  // LDS: [scale ring (MX only) | STAGES stages | 1 KB junk slot for zero DMA]
  static constexpr int SC_OFF = 0;                    // scale ring: 2 slots of SC_CHUNKS x 16 B
  static constexpr int SC_SLOT = SC_CHUNKS * 16;
  static constexpr int ST0 = 2 * SC_SLOT;             // first stage
  static constexpr int JUNK = ST0 + STAGES * STAGE_BYTES;
  static constexpr int RING_END = JUNK + 1024;
  static constexpr int LDS_BYTES = RING_END > Y_BYTES ? RING_END : Y_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  // chunk c of row r stored at c ^ swz(r): the 64-byte-row swizzle of the
  // bf16 A tile (the fragment read pattern is the same: 32 consecutive rows,
  // chunk h for lanes of half h, then chunk 2 + h)
  __host__ __device__ static constexpr int swz(int row) {
    return (((row >> 2) & 1) << 1) | (((row >> 1) ^ (row >> 3)) & 1);
  }
};

// SA, SW, ks: MXFP8 scales and their row stride (MX mode only; K % 64 == 0
// and ks % 16 == 0 there).
template <int MODE, int BM, int BNW, int STAGES, int WGM, int WGN>
__device__ __forceinline__ void f8_tile(const uint8_t* __restrict__ A,
                                        const uint8_t* __restrict__ W,
                                        uint16_t* __restrict__ Y, int M, int N, int K,
                                        float sg, float su, const uint8_t* __restrict__ SA,
                                        const uint8_t* __restrict__ SW, int ks, int m0, int tn,
                                        uint8_t* smem) {
  using C = F8Tiled<MODE, BM, BNW, STAGES, WGM, WGN>;
  static_assert(MODE == MODE_INTERLEAVE || MODE == MODE_SYNC || MODE == MODE_MX ||
                    MODE == MODE_MX_SYNC,
                "FP8 modes");
  constexpr bool kSync = C::SYNC;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int wr0 = tn * BNW;  // first W8 row of the tile (interleave)
  const int y0 = tn * C::BNY;
  // K steps: the sync mode runs them twice (Gate, then Up), its Gate phase
  // padded with zero steps to a ring boundary (nk0) so that the Up phase
  // starts on stage 0 with the same fragment-buffer parity -- in MX mode to a
  // scale-group boundary, so that its steps keep their positions in the
  // unrolled blocks
  const int nk = (K + C::BK - 1) / C::BK;
  const int nk0 = kSync ? (nk + C::UNR - 1) / C::UNR * C::UNR : nk;
  const int total = kSync ? nk0 + nk : nk;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // ---- DMA of one K step ----------------------------------------------------------
  // A chunk or a weight chunk is zero-filled when its row is out of range or
  // its k is (rows are k-contiguous, so a chunk past K would read the next
  // row: both sources check k).  All sums below stay under 2^32: offsets are
  // < 2^31 (tensors are smaller) and k0 <= K < 2^31.
  const i32x4 rsA = make_rsrc(A, (uint32_t)((size_t)M * K));
  const i32x4 rsW = make_rsrc(W, (uint32_t)((size_t)2 * N * K));
  const uint32_t lds0 = lds_addr(smem);
  constexpr uint32_t kRowOut = 0x80000000u;  // k of a chunk whose row is out of range
  uint32_t a_off[C::A_LOADS], a_k[C::A_LOADS];
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int p = tid + C::kThreads * i;
    const int row = p / 4;
    const int c = (p % 4) ^ C::swz(row);
    const bool in = m0 + row < M;
    a_off[i] = in ? (uint32_t)((size_t)(m0 + row) * K + c * 16) : 0u;
    a_k[i] = in ? (uint32_t)(c * 16) : kRowOut;
  }
  // weight tile row r: W8 row wr0 + r (interleave), or 2 (y0 + r) + phase (sync)
  uint32_t w_off[C::W_LOADS], w_k[C::W_LOADS];
#pragma unroll
  for (int i = 0; i < C::W_LOADS; ++i) {
    const int p = tid + C::kThreads * i;
    const int row = p / 4;
    const int c = (p % 4) ^ C::swz(row);
    const bool in = kSync ? y0 + row < N : wr0 + row < 2 * N;
    const size_t wrow = kSync ? 2 * (size_t)(y0 + row) : (size_t)(wr0 + row);
    w_off[i] = in ? (uint32_t)(wrow * K + c * 16) : 0u;
    w_k[i] = in ? (uint32_t)(c * 16) : kRowOut;
  }
  // MX: scale chunk p of the tile is row p of A's scales (p < BM) or the
  // scale row of weight tile row p - BM (W8 row wr0 + p - BM, or in the sync
  // order 2 (y0 + p - BM) for Gate and the next row for Up); group g of 8 K
  // steps is bytes [16 g, 16 g + 16) of the row.
  // The two-slot scale ring is indexed by a group count that runs on from the
  // Gate phase into the Up phase (the Up phase's first group takes the slot
  // the Gate phase's last group did not).
  const i32x4 rsSA = make_rsrc(SA, C::MX ? (uint32_t)((size_t)M * ks) : 0u);
  const i32x4 rsSW = make_rsrc(SW, C::MX ? (uint32_t)((size_t)2 * N * ks) : 0u);
  const int ngroups = (nk + 7) / 8;  // scale groups of one phase
  uint32_t sc_off[C::SC_LOADS > 0 ? C::SC_LOADS : 1];
#pragma unroll
  for (int i = 0; i < C::SC_LOADS; ++i) {
    const int p = tid + C::kThreads * i;
    const bool in = p < BM ? m0 + p < M : (kSync ? y0 + (p - BM) < N : wr0 + (p - BM) < 2 * N);
    const size_t row = p < BM ? (size_t)(m0 + p)
                              : (kSync ? 2 * (size_t)(y0 + p - BM) : (size_t)(wr0 + p - BM));
    sc_off[i] = in ? (uint32_t)(row * ks) : kOutOfRange;
  }
  // DMA instruction q (A chunks first, then weight chunks, then in MX mode the
  // scale chunk) of K step `it` into stage ST; padding steps and steps past
  // the end load zeros (k0 = K)
  auto dma = [&](int it, auto st_c, int q) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    const bool up = kSync && it >= nk0;
    const int kt = up ? it - nk0 : it;
    const uint32_t k0 = (it < total && kt < nk) ? (uint32_t)kt * C::BK : (uint32_t)K;
    const uint32_t sbase = lds0 + C::ST0 + ST * C::STAGE_BYTES;
    if (q < C::A_LOADS) {
      const int p0 = C::kThreads * q + 64 * wave_u;
      const bool own = p0 < C::A_CHUNKS;
      const uint32_t off = (own && k0 + a_k[q] < (uint32_t)K) ? a_off[q] + k0 : kOutOfRange;
      lds_dma16(own ? sbase + p0 * 16 : lds0 + C::JUNK, off, rsA);
    } else if (q < C::LOADS) {
      const int i = q - C::A_LOADS;
      const int p0 = C::kThreads * i + 64 * wave_u;
      const bool own = p0 < C::W_CHUNKS;
      const uint32_t off = (own && k0 + w_k[i] < (uint32_t)K)
                               ? w_off[i] + (up ? (uint32_t)K : 0u) + k0
                               : kOutOfRange;
      lds_dma16(own ? sbase + C::A_BYTES + p0 * 16 : lds0 + C::JUNK, off, rsW);
    } else if constexpr (C::MX) {
      // the scale chunks of group kt / 8 of the phase with step kt of a group
      // start, else nothing
      const int i = q - C::LOADS;
      const int p0 = C::kThreads * i + 64 * wave_u;
      const bool own = p0 < C::SC_CHUNKS;
      const bool real = own && (kt & 7) == 0 && kt < nk && it < total;
      const int g = kt >> 3;
      const int slot = (up ? ngroups + g : g) & 1;
      const uint32_t wrow = (up && p0 >= BM) ? (uint32_t)ks : 0u;  // Up: the next W8 row
      const uint32_t off = (real && sc_off[i] != kOutOfRange)
                               ? sc_off[i] + wrow + (uint32_t)(16 * g)
                               : kOutOfRange;
      const uint32_t dst = real ? lds0 + C::SC_OFF + slot * C::SC_SLOT + p0 * 16
                                : lds0 + C::JUNK;
      lds_dma16(dst, off, p0 < BM ? rsSA : rsSW);
    }
  };

  // ---- fragments ------------------------------------------------------------------
  const int h = lane >> 5;
  const int a_row = wm * C::WTM + (lane & 31);  // + 32 fa
  const int w_row = wn * C::WTW + (lane & 31);  // + 32 fw
  // The swizzle depends on row bits 1-3 only, so the rows +32, +64, ... of a
  // lane's fragments share it: one pair of per-lane offsets per tile, the
  // fragment index a compile-time displacement of 32 rows.
  // Offsets from the LDS base: an LDS read adds at most 65535 to its address
  // register, so the stages above 64 KB read through a second copy of each
  // offset raised by 64 KB, which the compiler cannot see through (an empty
  // asm statement).  Otherwise it formed one address register per stage and
  // fragment (the largest tile then spilled).
  int frag_off[2][4];  // [window][a_lo, a_hi, w_lo, w_hi]
  frag_off[0][0] = a_row * C::BK + ((h ^ C::swz(a_row)) * 16);
  frag_off[0][1] = a_row * C::BK + (((2 + h) ^ C::swz(a_row)) * 16);
  frag_off[0][2] = C::A_BYTES + w_row * C::BK + ((h ^ C::swz(w_row)) * 16);
  frag_off[0][3] = C::A_BYTES + w_row * C::BK + (((2 + h) ^ C::swz(w_row)) * 16);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    int hi = frag_off[0][v] + 65536;
    asm volatile("" : "+v"(hi));
    frag_off[1][v] = hi;
  }
  // fragment f of the A tile (f < FA) or of the weight tile (W) in stage ST
  auto frag_read = [&](auto st_c, int v, int f) __attribute__((always_inline)) -> u32x4 {
    constexpr int BASE = C::ST0 + decltype(st_c)::value * C::STAGE_BYTES;
    constexpr int WIN = BASE >= 65536 ? 1 : 0;
    return *reinterpret_cast<const u32x4*>(smem + frag_off[WIN][v] + (BASE - WIN * 65536) +
                                           f * 32 * C::BK);
  };
  auto readA = [&](auto st_c, int f, u32x4 (&d)[2]) __attribute__((always_inline)) {
    d[0] = frag_read(st_c, 0, f);
    d[1] = frag_read(st_c, 1, f);
  };
  auto readW = [&](auto st_c, int f, u32x4 (&d)[2]) __attribute__((always_inline)) {
    d[0] = frag_read(st_c, 2, f);
    d[1] = frag_read(st_c, 3, f);
  };
  u32x4 wf[C::FW][2];
  u32x4 af[2][C::FA][2];
  // MX: scale bytes of the lane's rows, packed (the MFMA selects a byte):
  // weight block i in byte i of scw[P], activation block j in byte j of
  // sca[P], for the steps of parity P.  The bytes of the next step are read
  // into scn during a step and packed after its last MFMA: no VALU write to
  // a scale register then falls between the MFMAs that read it, and the LDS
  // byte reads are waited for where the step's fragment reads are anyway.
  static_assert(!C::MX || (C::FW <= 4 && C::FA <= 4), "packed scale bytes");
  uint32_t scw[2] = {0u, 0u}, sca[2] = {0u, 0u};
  uint32_t scn[C::MX ? C::FA + C::FW : 1];
  auto pack_scales = [&](uint32_t& a, uint32_t& w) __attribute__((always_inline)) {
    a = 0u, w = 0u;
#pragma unroll
    for (int j = 0; j < C::FA; ++j) a |= scn[j] << (8 * j);
#pragma unroll
    for (int i = 0; i < C::FW; ++i) w |= scn[C::FA + i] << (8 * i);
  };
  // Step s (kt the step within its phase) takes block 2 kt + h of each row's
  // scales (h: this lane's fragment half): byte 2 (kt % 8) + h of the row's
  // chunk of group kt / 8.  In MX mode kt % 8 is the step's position in the
  // unrolled block, a compile-time constant, so a scale read is a per-lane
  // row base, a wave-uniform ring slot and an immediate.
  const int sca_base = a_row * 16 + h;         // + 512 q for activation fragment q
  const int scw_base = (BM + w_row) * 16 + h;  // + 512 i for weight fragment i
  auto scale_slot = [&](int s) __attribute__((always_inline)) -> int {
    const bool up = kSync && s >= nk0;
    const int kt = up ? s - nk0 : s;
    const int g = up ? ngroups + (kt >> 3) : (kt >> 3);
    return C::SC_OFF + (g & 1) * C::SC_SLOT;
  };
  auto scale_at = [&](int slot, int base, int imm) __attribute__((always_inline)) -> uint32_t {
    return smem[slot + base + imm];
  };
  f32x16 acc[C::NACC][C::FW][C::FA];
#pragma unroll
  for (int p = 0; p < C::NACC; ++p)
#pragma unroll
    for (int i = 0; i < C::FW; ++i)
#pragma unroll
      for (int j = 0; j < C::FA; ++j) acc[p][i][j] = f32x16{};

  // One K step on stage ST.  After the barrier, every wave has the loads of
  // step it+1 in LDS and has finished reading stage ST, so the MFMAs of step
  // `it` run beside the fragment reads of step it+1 (stage ST+1) and the DMA
  // of step it+STAGES into stage ST.
  constexpr int NMF = C::FW * C::FA;
  constexpr int DBEGIN = NMF / 2;
  constexpr int DSLOTS = NMF - DBEGIN;
  auto kstep = [&](int it, auto st_c, auto phase_c, auto pos_c) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    constexpr int PH = decltype(phase_c)::value;
    constexpr int T = decltype(pos_c)::value;  // position in the unrolled block
    constexpr int P = ST & 1;
    constexpr int TL = C::step_loads(T + STAGES);  // DMA instructions of step it + STAGES
    constexpr int NB = 2 * ((T + 1) % 8);            // the next step's byte in its group's chunk
    using Next = std::integral_constant<int, (ST + 1) % STAGES>;
    wait_vmcnt<C::in_flight(T)>();
    __syncthreads();
    const int nslot = C::MX ? scale_slot(it + 1) : 0;
    // the sync order's Gate padding steps (zero tiles) take scale 1 (byte
    // 127) whatever a scale row holds past K / 32: a NaN code there (255)
    // would turn their zero products into NaN
    const bool npad = kSync && it + 1 >= nk && it + 1 < nk0;
    // MFMA slot q (compile time): MFMA (i, j), then its share of the reads of
    // step it+1 and of the DMA of step it+STAGES
    auto slot = [&](auto q_c) __attribute__((always_inline)) {
      constexpr int q = decltype(q_c)::value;
      constexpr int i = q / C::FA, j = q % C::FA;
      if constexpr (C::MX)
        acc[PH][i][j] = mfma32_f8_scaled<i, j>(wf[i], af[P][j], acc[PH][i][j], scw[P], sca[P]);
      else
        acc[PH][i][j] = mfma32_f8(wf[i], af[P][j], acc[PH][i][j]);
      if constexpr (q < C::FA) {
        readA(Next{}, q, af[P ^ 1][q]);
        if constexpr (C::MX) scn[q] = scale_at(nslot, sca_base, 512 * q + NB);
      }
      if constexpr (j == C::FA - 1) {
        readW(Next{}, i, wf[i]);
        if constexpr (C::MX) scn[C::FA + i] = scale_at(nslot, scw_base, 512 * i + NB);
      }
      if constexpr (q >= DBEGIN) {
#pragma unroll
        for (int x = (q - DBEGIN) * TL / DSLOTS; x < (q - DBEGIN + 1) * TL / DSLOTS; ++x)
          dma(it + STAGES, st_c, x);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    [&]<int... Q>(std::integer_sequence<int, Q...>) __attribute__((always_inline)) {
      (slot(std::integral_constant<int, Q>{}), ...);
    }(std::make_integer_sequence<int, NMF>{});
    if constexpr (C::MX) {
      pack_scales(sca[P ^ 1], scw[P ^ 1]);
      if (npad) sca[P ^ 1] = scw[P ^ 1] = 0x7f7f7f7fu;
    }
  };
  // steps [b, e) with b on a block boundary: whole unrolled blocks (stage
  // rings, or MX scale groups), then the rest
  auto run = [&](int b, int e, auto phase_c) __attribute__((always_inline)) {
    int it = b;
    for (; it + C::UNR <= e; it += C::UNR)
      [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
        (kstep(it + S, std::integral_constant<int, S % STAGES>{}, phase_c,
               std::integral_constant<int, S>{}),
         ...);
      }(std::make_integer_sequence<int, C::UNR>{});
    [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
      ((it + S < e ? (kstep(it + S, std::integral_constant<int, S % STAGES>{}, phase_c,
                            std::integral_constant<int, S>{}),
                      0)
                   : 0),
       ...);
    }(std::make_integer_sequence<int, C::UNR - 1>{});
  };

  // ---- prologue: steps 0 .. STAGES-1 in flight, fragments of step 0 --------------
  [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
    ((
         [&] {
#pragma unroll
           for (int q = 0; q < C::step_loads(S); ++q) dma(S, std::integral_constant<int, S>{}, q);
         }()),
     ...);
  }(std::make_integer_sequence<int, STAGES>{});
  wait_vmcnt<C::prologue_in_flight()>();
  __syncthreads();
#pragma unroll
  for (int j = 0; j < C::FA; ++j) {
    readA(std::integral_constant<int, 0>{}, j, af[0][j]);
    if constexpr (C::MX) scn[j] = scale_at(scale_slot(0), sca_base, 512 * j);
  }
#pragma unroll
  for (int i = 0; i < C::FW; ++i) {
    readW(std::integral_constant<int, 0>{}, i, wf[i]);
    if constexpr (C::MX) scn[C::FA + i] = scale_at(scale_slot(0), scw_base, 512 * i);
  }
  if constexpr (C::MX) pack_scales(sca[0], scw[0]);

  if constexpr (kSync) {
    run(0, nk0, std::integral_constant<int, 0>{});
    // Gate finished: scale and SiLU in registers while Up tiles are in flight
#pragma unroll
    for (int i = 0; i < C::FW; ++i)
#pragma unroll
      for (int j = 0; j < C::FA; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[0][i][j][r] = silu(sg * acc[0][i][j][r]);
    run(nk0, total, std::integral_constant<int, 1>{});
  } else {
    run(0, total, std::integral_constant<int, 0>{});
  }

  // ---- epilogue: scales, SiLU(Gate) * Up, bf16 tile through LDS, row stores -------
  wait_vmcnt<0>();
  __syncthreads();
  // The lane's epilogue offsets come from a copy of the thread index the
  // compiler cannot see through (an empty asm statement): otherwise they were
  // computed before the K loop and kept live through it, where the largest
  // tile needs every register, and spilled to scratch.
  int etid = threadIdx.x;
  asm volatile("" : "+v"(etid));
  const int e_lane = etid & 63, e_wave = etid >> 6;
  const int e_row = (e_wave / WGN) * C::WTM + (e_lane & 31);
  const int e_wcl = (e_wave % WGN) * C::WTW + 4 * (e_lane >> 5);
  uint16_t* ys = reinterpret_cast<uint16_t*>(smem);  // [BM][YLD]
#pragma unroll
  for (int i = 0; i < C::FW; ++i)
#pragma unroll
    for (int j = 0; j < C::FA; ++j) {
      const int row = e_row + j * 32;
      const f32x16& d = acc[0][i][j];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // registers 4q..4q+3: weight tile rows wcl..wcl+3
        const int wcl = e_wcl + i * 32 + 8 * q;
        if constexpr (kSync) {
          // output columns wcl..wcl+3: SiLU(Gate) (already applied) * Up
          const f32x16& u = acc[C::NACC - 1][i][j];
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = d[4 * q + e] * (su * u[4 * q + e]);
          *reinterpret_cast<u32x2*>(ys + row * C::YLD + wcl) =
              u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        } else {
          // W8 rows wcl..wcl+3 = Gate/Up of output columns wcl/2, wcl/2+1
          const float ya = silu(sg * d[4 * q + 0]) * (su * d[4 * q + 1]);
          const float yb = silu(sg * d[4 * q + 2]) * (su * d[4 * q + 3]);
          *reinterpret_cast<uint32_t*>(ys + row * C::YLD + wcl / 2) = pack_bf16x2(ya, yb);
        }
      }
    }
  __syncthreads();
  constexpr int YCH = C::BNY / 8;
  for (int p = tid; p < BM * YCH; p += C::kThreads) {
    const int row = p / YCH, cq = p % YCH;
    const int gr = m0 + row, gc = y0 + cq * 8;
    if (gr < M && gc < N)
      *reinterpret_cast<u32x4*>(Y + (size_t)gr * N + gc) =
          *reinterpret_cast<const u32x4*>(ys + row * C::YLD + cq * 8);
  }
}

template <int MODE, int BM, int BNW, int STAGES, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void f8_kernel(const uint8_t* __restrict__ A,
                                                             const uint8_t* __restrict__ W,
                                                             uint16_t* __restrict__ Y, int M,
                                                             int N, int K, float sg, float su,
                                                             const uint8_t* __restrict__ SA,
                                                             const uint8_t* __restrict__ SW,
                                                             int ks, int group_m) {
  using C = F8Tiled<MODE, BM, BNW, STAGES, WGM, WGN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];
  const int ntm = (M + BM - 1) / BM;
  const int ntn = (N + C::BNY - 1) / C::BNY;
  int tm, tn;
  tile_of(xcd_remap(blockIdx.x, gridDim.x), ntm, ntn, group_m, tm, tn);
  f8_tile<MODE, BM, BNW, STAGES, WGM, WGN>(A, W, Y, M, N, K, sg, su, SA, SW, ks, tm * BM, tn,
                                           smem);
}

// The split tail of tiled_split_kernel for the FP8 tiles: workgroups
// [0, n_big) take whole tiles, the rest quarter tiles of the partial last round.
template <int MODE, int BM, int BNW, int STAGES, int WGM, int WGN, int SWGM, int SWGN>
__global__ __launch_bounds__(64 * WGM * WGN) void f8_split_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, uint16_t* __restrict__ Y,
    int M, int N, int K, float sg, float su, const uint8_t* __restrict__ SA,
    const uint8_t* __restrict__ SW, int ks, int group_m, int n_big) {
  using Big = F8Tiled<MODE, BM, BNW, STAGES, WGM, WGN>;
  using Small = F8Tiled<MODE, BM / 2, BNW / 2, STAGES, SWGM, SWGN>;
  static_assert(Big::kThreads == Small::kThreads, "one workgroup size for both tile kinds");
  constexpr int LDS = Big::LDS_BYTES > Small::LDS_BYTES ? Big::LDS_BYTES : Small::LDS_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];
  const int ntm = (M + BM - 1) / BM;
  const int ntn = (N + Big::BNY - 1) / Big::BNY;
  int tm, tn;
  if ((int)blockIdx.x < n_big) {
    tile_of(xcd_remap(blockIdx.x, n_big), ntm, ntn, group_m, tm, tn);
    f8_tile<MODE, BM, BNW, STAGES, WGM, WGN>(A, W, Y, M, N, K, sg, su, SA, SW, ks, tm * BM, tn,
                                             smem);
  } else {
    const int u = blockIdx.x - n_big, q = u & 3;
    tile_of(n_big + u / 4, ntm, ntn, group_m, tm, tn);
    const int m0 = tm * BM + (q >> 1) * (BM / 2);
    const int tq = 2 * tn + (q & 1);
    if (m0 >= M || tq * Small::BNY >= N) return;
    f8_tile<MODE, BM / 2, BNW / 2, STAGES, SWGM, SWGN>(A, W, Y, M, N, K, sg, su, SA, SW, ks, m0,
                                                       tq, smem);
  }
}

// FP8 weight streaming for decode-sized batches (M <= 16 MT): split-K over
// the waves of a workgroup, v_mfma_scale_f32_16x16x128_f8f6f4 with unit block
// scales.  W8 is k-contiguous, so a weight fragment (16 W8 rows x 128 k) is
// two plain 16-byte loads per lane straight from HBM into the MFMA source
// registers -- no transposition, no LDS.  Lane l takes row l%16 and the
// 16-byte chunks l/16 and 4 + l/16 of the step (one instruction reads 64
// contiguous bytes of each row), the same for the activation rows.  Each
// wave keeps the next step's loads in flight while it multiplies; the fp32
// partial sums of the waves are added through LDS in a fixed order before
// the scales and SiLU (the activation needs the complete sum).
template <int MT, int NB, int NW>
struct F8Skinny {
  static constexpr int kThreads = 64 * NW;
  static constexpr int SLAB_W = 16 * NB;  // W8 rows per workgroup
  static constexpr int SLAB_Y = SLAB_W / 2;
  static constexpr int LDS_BYTES = NW * MT * NB * 64 * 16;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

template <int MT, int NB, int NW>
__global__ __launch_bounds__(64 * NW) void f8_skinny_kernel(const uint8_t* __restrict__ A,
                                                             const uint8_t* __restrict__ W,
                                                             uint16_t* __restrict__ Y, int M,
                                                             int N, int K, float sg,
                                                             float su) {
  using C = F8Skinny<MT, NB, NW>;
  __shared__ __attribute__((aligned(16))) f32x4 red[NW * MT * NB * 64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slab = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = blockIdx.y * MT * 16;
  const int r16 = lane & 15, g = lane >> 4;

  const int nsteps = (K + 127) / 128;
  const int per = (nsteps + NW - 1) / NW;
  const int s_begin = wave * per;
  const int s_end = min(nsteps, s_begin + per);

  // byte offsets of this lane's rows (k = 0); rows out of range load zeros
  const int wrow0 = slab * C::SLAB_W + r16;
  f32x4 acc[MT][NB];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[mt][b] = f32x4{};

  auto load = [&](int s, u32x4 (&wv)[NB][2], u32x4 (&av)[MT][2]) __attribute__((always_inline)) {
    const int k0 = s * 128 + 16 * g, k1 = k0 + 64;
    const bool in0 = k0 < K, in1 = k1 < K;  // K % 16 == 0: chunks are whole
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int row = wrow0 + 16 * b;
      const bool ok = row < 2 * N;
      const uint8_t* p = W + (size_t)row * K;
      const u32x4 z{0, 0, 0, 0};
      wv[b][0] = (ok && in0) ? (MT == 1 ? load16_stream(p + k0) : load16(p + k0)) : z;
      wv[b][1] = (ok && in1) ? (MT == 1 ? load16_stream(p + k1) : load16(p + k1)) : z;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + mt * 16 + r16;
      const bool ok = m < M;
      const uint8_t* p = A + (size_t)m * K;
      av[mt][0] = (ok && in0) ? load16(p + k0) : u32x4{0, 0, 0, 0};
      av[mt][1] = (ok && in1) ? load16(p + k1) : u32x4{0, 0, 0, 0};
    }
  };
  auto mma = [&](const u32x4 (&wv)[NB][2], const u32x4 (&av)[MT][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt][b] = mfma16_f8(wv[b], av[mt], acc[mt][b]);
  };

  // two register sets: the loads of step s+1 are in flight while step s multiplies
  u32x4 wa[NB][2], aa[MT][2], wb[NB][2], ab[MT][2];
  int s = s_begin;
  if (s < s_end) load(s, wa, aa);
  for (; s < s_end; s += 2) {
    if (s + 1 < s_end) load(s + 1, wb, ab);
    mma(wa, aa);
    if (s + 1 >= s_end) break;
    if (s + 2 < s_end) load(s + 2, wa, aa);
    mma(wb, ab);
  }

  // ---- split-K reduction through LDS (fixed order: wave 0, 1, ..., NW-1) ----
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int b = 0; b < NB; ++b) red[((wave * MT + mt) * NB + b) * 64 + lane] = acc[mt][b];
  __syncthreads();
  for (int q = wave; q < MT * NB; q += NW) {
    const int mt = q / NB, b = q % NB;
    f32x4 v = red[(mt * NB + b) * 64 + lane];
    for (int w = 1; w < NW; ++w) v += red[((w * MT + mt) * NB + b) * 64 + lane];
    // lane: A row r16 of the block, W8 rows 4g..4g+3 = (Gate, Up) of two columns
    const int row = m0 + mt * 16 + r16;
    const int col = slab * C::SLAB_Y + 8 * b + 2 * g;
    if (row < M && col < N) {
      const float y0 = silu(sg * v[0]) * (su * v[1]);
      const float y1 = silu(sg * v[2]) * (su * v[3]);
      *reinterpret_cast<uint32_t*>(Y + (size_t)row * N + col) = pack_bf16x2(y0, y1);
    }
  }
}

// FP8 streaming on fragment-ordered W8: the layout of packed_kernel carried
// over to the E4M3 k-major pairing.  W8 [2N, K] (row 2n Gate, 2n+1 Up) is cut
// into blocks of 16 rows and steps of 128 k; block (rb, t) is 2 KB, the B
// operand of one v_mfma_scale_f32_16x16x128_f8f6f4 for all 64 lanes, stored
// as two 1 KB halves:
//   P8[((rb T + t) 2 + h) 1024 + (16 g + i) 16 + e] = W8[16 rb + i][128 t + 64 h + 16 g + e]
// with T = ceil(K / 128), h < 2, g < 4, i, e < 16, zeros past 2N and K.  Lane
// 16 g + i reads 16 bytes of each half, so every load instruction reads 1 KB
// contiguous and a row block is one contiguous span over K.  The workgroup
// (NB row blocks, NW waves taking the steps in turn), the two register sets,
// the LDS reduction in wave order and the epilogue are those of
// f8_skinny_kernel; as in packed_kernel every load is issued unconditionally
// (clamped addresses, k past K zeroed right before the MFMAs) so that the
// in-order load counter stays exact.
template <int MT, int NB, int NW>
struct F8Packed {
  static constexpr int kThreads = 64 * NW;
  static constexpr int LDS_BYTES = NW * MT * NB * 64 * 16;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static constexpr int SLAB_W = 16 * NB;  // W8 rows per workgroup
  static constexpr int SLAB_Y = 8 * NB;   // output columns per workgroup
};

template <int MT, int NB, int NW>
__global__ __launch_bounds__(64 * NW) void f8_packed_kernel(const uint8_t* __restrict__ A,
                                                            const uint8_t* __restrict__ P,
                                                            uint16_t* __restrict__ Y, int M,
                                                            int N, int K, float sg, float su) {
  using C = F8Packed<MT, NB, NW>;
  __shared__ __attribute__((aligned(16))) f32x4 red[NW * MT * NB * 64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = blockIdx.y * MT * 16;
  const int r16 = lane & 15, g = lane >> 4;
  const int nsteps = (K + 127) / 128;
  const int nrb = (2 * N + 15) / 16;  // row blocks in P8 (padding included)

  // this lane's 16 bytes in the first half of each of the workgroup's row
  // blocks; a block past the last one re-reads it (its outputs are past N)
  const uint8_t* wp[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    wp[b] = P + (size_t)min(unit * NB + b, nrb - 1) * (size_t)nsteps * 2048 + lane * 16;

  f32x4 acc[MT][NB];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[mt][b] = f32x4{};

  auto load = [&](int s, u32x4 (&wv)[NB][2], u32x4 (&av)[MT][2]) __attribute__((always_inline)) {
    // activations: rows past M re-read row M-1 (never stored), k past K
    // re-reads the last 16 bytes (zeroed by mma); K % 16 == 0, K >= 16
    const int k0 = min(s * 128 + 16 * g, K - 16), k1 = min(s * 128 + 64 + 16 * g, K - 16);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint8_t* p = A + (size_t)min(m0 + mt * 16 + r16, M - 1) * K;
      av[mt][0] = load16(p + k0);
      av[mt][1] = load16(p + k1);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint8_t* p = wp[b] + (size_t)s * 2048;
      wv[b][0] = MT == 1 ? load16_stream(p) : load16(p);
      wv[b][1] = MT == 1 ? load16_stream(p + 1024) : load16(p + 1024);
    }
  };
  auto mma = [&](const u32x4 (&wv)[NB][2], const u32x4 (&av)[MT][2], int s)
      __attribute__((always_inline)) {
    const bool in0 = s * 128 + 16 * g < K, in1 = s * 128 + 64 + 16 * g < K;
    const u32x4 z{0, 0, 0, 0};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 a[2] = {in0 ? av[mt][0] : z, in1 ? av[mt][1] : z};
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[mt][b] = mfma16_f8(wv[b], a, acc[mt][b]);
    }
  };

  // steps wave, wave + NW, ...: pairs loaded together (the scheduling
  // barriers keep both steps' loads ahead of the MFMAs and the two MFMA
  // groups apart), then an odd last one.  At the 7B decode shape this form
  // measured 23.6 us against 24.8 us software-pipelined and 24.5 us with no
  // barriers (one box).
  {
    u32x4 wa[NB][2], aa[MT][2], wb[NB][2], ab[MT][2];
    int s = wave;
    for (; s + NW < nsteps; s += 2 * NW) {
      load(s, wa, aa);
      load(s + NW, wb, ab);
      __builtin_amdgcn_sched_barrier(0);
      mma(wa, aa, s);
      __builtin_amdgcn_sched_barrier(0);
      mma(wb, ab, s + NW);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (s < nsteps) {
      load(s, wa, aa);
      mma(wa, aa, s);
    }
  }

  // ---- split-K reduction through LDS (fixed order: wave 0, 1, ..., NW-1) ----
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int b = 0; b < NB; ++b) red[((wave * MT + mt) * NB + b) * 64 + lane] = acc[mt][b];
  __syncthreads();
  for (int q = wave; q < MT * NB; q += NW) {
    const int mt = q / NB, b = q % NB;
    f32x4 v = red[(mt * NB + b) * 64 + lane];
    for (int w = 1; w < NW; ++w) v += red[((w * MT + mt) * NB + b) * 64 + lane];
    // lane: A row r16 of the block, W8 rows 4g..4g+3 = (Gate, Up) of two columns
    const int row = m0 + mt * 16 + r16;
    const int col = unit * C::SLAB_Y + 8 * b + 2 * g;
    if (row < M && col < N) {
      const float y0 = silu(sg * v[0]) * (su * v[1]);
      const float y1 = silu(sg * v[2]) * (su * v[3]);
      *reinterpret_cast<uint32_t*>(Y + (size_t)row * N + col) = pack_bf16x2(y0, y1);
    }
  }
}

// MXFP8 streaming on fragment-ordered W8, for M <= 32 per row group: the
// layout of the 32x32x64 scaled MFMA's sources.  W8 [2N, K] (row 2n Gate, 2n+1
// Up) is cut into blocks of 32 rows and steps of 64 k; block (rb, t) is 2 KB,
// stored as two 1 KB halves (the lanes' bytes 0-15, then 16-31):
//   P8[((rb T + t) 2 + v) 1024 + (i + 32 h) 16 + e] = W8[32 rb + i][64 t + 32 v + 16 h + e]
// with T = K / 64, v, h < 2, i < 32, e < 16, zeros past 2N.  Half v holds k
// block 2t + v of every row, so lane i + 32 h passes the scale of its row for
// block 2t + h (the instruction's convention for both sources), read straight
// from the E8M0 scale rows SW [2N, ks] and SA [M, ks]: 32 bytes per row cover
// 16 steps.  NW waves per workgroup stream NB row blocks; each wave takes a
// contiguous range of whole 16-step groups (NW = 1: all of K, no reduction;
// NW > 1 for narrow N, the fp32 partials then added through LDS in wave order
// before SiLU); the next step's loads are in flight while a step multiplies.
// Output: lane l holds A row l % 32 and W8 rows 8 (r/4) + 4 (l/32) + r % 4
// of register r, so (Gate, Up) pairs are adjacent registers.
template <int NB, int NW>
struct MxPacked {
  static constexpr int kThreads = 64 * NW;
  static constexpr int LDS_BYTES = NW > 1 ? NW * NB * 16 * 64 * 4 : 0;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static constexpr int SLAB_W = 32 * NB;  // W8 rows per workgroup
  static constexpr int SLAB_Y = 16 * NB;  // output columns per workgroup
};

template <int NB, int NW>
__global__ __launch_bounds__(64 * NW) void mx_packed_kernel(const uint8_t* __restrict__ A,
                                                            const uint8_t* __restrict__ SA,
                                                            const uint8_t* __restrict__ P,
                                                            const uint8_t* __restrict__ SW,
                                                            uint16_t* __restrict__ Y, int M,
                                                            int N, int K, int ks) {
  using C = MxPacked<NB, NW>;
  __shared__ __attribute__((aligned(16))) float red[NW > 1 ? NW * NB * 16 * 64 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = blockIdx.y * 32;
  const int i32 = lane & 31, h = lane >> 5;
  const int nsteps = K / 64;              // K % 64 == 0
  const int nrb = (2 * N + 31) / 32;      // row blocks in P8 (padding included)
  const int R = 2 * N;
  // this wave's groups of 16 steps: [g0, g1), steps [16 g0, s1)
  const int ngroups = (nsteps + 15) / 16;
  const int g0 = wave * ngroups / NW, g1 = (wave + 1) * ngroups / NW;
  const int s1 = min(16 * g1, nsteps);

  // this lane's 16 bytes of half 0 of each of the workgroup's row blocks (a
  // block past the last re-reads it; its outputs are past N), its A row
  // (rows past M re-read row M-1, never stored), and its scale rows
  const uint8_t* wp[NB];
  const uint8_t* swr[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int rb = min(unit * NB + b, nrb - 1);
    wp[b] = P + (size_t)rb * (size_t)nsteps * 2048 + lane * 16;
    swr[b] = SW + (size_t)min(32 * rb + i32, R - 1) * ks;
  }
  const int arow = min(m0 + i32, M - 1);
  const uint8_t* ap = A + (size_t)arow * K + 16 * h;
  const uint8_t* sar = SA + (size_t)arow * ks;

  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x16{};

  // scale bytes of 16 steps: row bytes [32 g, 32 g + 32) as two 16-byte
  // chunks; a chunk at or past ks (its blocks lie past K) re-reads the last
  // (ks % 16 == 0, ks >= K / 32 >= 2)
  auto load_scales = [&](const uint8_t* row, int g, u32x4 (&sc)[2]) __attribute__((always_inline)) {
    sc[0] = load16(row + min(32 * g, ks - 16));
    sc[1] = load16(row + min(32 * g + 16, ks - 16));
  };
  // scale of step j (0..15) of a group for this lane's block 2t + h: byte
  // 2 (j % 8) + h of chunk j / 8, moved to the low byte
  auto pick = [&](const u32x4 (&sc)[2], int j) __attribute__((always_inline)) {
    const uint32_t w = sc[j >> 3][(j & 7) >> 1];
    return w >> (8 * (2 * (j & 1) + h));
  };
  auto load = [&](int t, u32x4 (&wv)[NB][2], u32x4 (&av)[2]) __attribute__((always_inline)) {
    av[0] = load16(ap + (size_t)t * 64);
    av[1] = load16(ap + (size_t)t * 64 + 32);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint8_t* p = wp[b] + (size_t)t * 2048;
      wv[b][0] = load16_stream(p);
      wv[b][1] = load16_stream(p + 1024);
    }
  };

  // scales of the next group are loaded a group ahead, so no step waits for
  // them (a group past the end re-reads in-bounds bytes, unused)
  u32x4 wa[NB][2], aa[2], wb[NB][2], ab[2];
  u32x4 sw_c[NB][2], sa_c[2], sw_n[NB][2], sa_n[2];
  if (g0 < g1) {
#pragma unroll
    for (int b = 0; b < NB; ++b) load_scales(swr[b], g0, sw_n[b]);
    load_scales(sar, g0, sa_n);
    load(16 * g0, wa, aa);
  }
  for (int g = g0; g < g1; ++g) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      sw_c[b][0] = sw_n[b][0];
      sw_c[b][1] = sw_n[b][1];
      load_scales(swr[b], g + 1, sw_n[b]);
    }
    sa_c[0] = sa_n[0];
    sa_c[1] = sa_n[1];
    load_scales(sar, g + 1, sa_n);
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const int t = 16 * g + j;
      if (t >= s1) break;
      load(min(t + 1, s1 - 1), wb, ab);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = mfma32_f8_scaled<0, 0>(wa[b], aa, acc[b], pick(sw_c[b], j), pick(sa_c, j));
      if (t + 1 >= s1) break;
      load(min(t + 2, s1 - 1), wa, aa);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = mfma32_f8_scaled<0, 0>(wb[b], ab, acc[b], pick(sw_c[b], j + 1),
                                        pick(sa_c, j + 1));
    }
  }

  if constexpr (NW > 1) {
    // split-K reduction through LDS (fixed order: wave 0, 1, ..., NW-1);
    // wave 0 finishes
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((wave * NB + b) * 16 + r) * 64 + lane] = acc[b][r];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = red[(b * 16 + r) * 64 + lane];
        for (int w = 1; w < NW; ++w) v += red[((w * NB + b) * 16 + r) * 64 + lane];
        acc[b][r] = v;
      }
  }

  // epilogue: registers (4q, 4q+1) and (4q+2, 4q+3) are (Gate, Up) pairs of
  // W8 rows 8q + 4h + {0,1} and {2,3}: output columns of this lane's A row
  const int row = m0 + i32;
  if (row >= M) return;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = unit * C::SLAB_Y + 16 * b + 4 * q + 2 * h;  // (W8 row) / 2
      if (col < N) {
        const float y0 = silu(acc[b][4 * q]) * acc[b][4 * q + 1];
        const float y1 = silu(acc[b][4 * q + 2]) * acc[b][4 * q + 3];
        *reinterpret_cast<uint32_t*>(Y + (size_t)row * N + col) = pack_bf16x2(y0, y1);
      }
    }
  }
}

// Fragment-ordered W8 for the MXFP8 streaming kernel from W8 [R = 2N, K]
// (layout in front of mx_packed_kernel): a thread copies one 16-byte chunk,
// row 32 rb + i, bytes [64 t + 32 v + 16 h, +16), zeros past R.  Once per
// weight set.
__global__ __launch_bounds__(256) void pack_mx_frag_kernel(const uint8_t* __restrict__ W8,
                                                           uint8_t* __restrict__ P, int R, int K,
                                                           size_t nchunks) {
  const int nsteps = K / 64;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks;
       c += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(c & 63);
    const int v = (int)((c >> 6) & 1);
    const size_t bt = c >> 7;  // rb * nsteps + t
    const int t = (int)(bt % (size_t)nsteps);
    const long long rb = (long long)(bt / (size_t)nsteps);
    const long long r = 32 * rb + (lane & 31);
    const int k0 = 64 * t + 32 * v + 16 * (lane >> 5);
    u32x4 x{0, 0, 0, 0};
    if (r < R) x = load16(W8 + (size_t)r * (size_t)K + k0);  // K % 64 == 0
    *reinterpret_cast<u32x4*>(P + c * 16) = x;
  }
}

// Fragment-ordered W8 from W8 [R = 2N, K] (layout in front of
// f8_packed_kernel): a thread copies one 16-byte chunk, row 16 rb + i, bytes
// [128 t + 64 h + 16 g, +16), zeros past R and K.  Once per weight set.
__global__ __launch_bounds__(256) void pack_f8_frag_kernel(const uint8_t* __restrict__ W8,
                                                           uint8_t* __restrict__ P, int R, int K,
                                                           size_t nchunks) {
  const int nsteps = (K + 127) / 128;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nchunks;
       i += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63);
    const int h = (int)((i >> 6) & 1);
    const size_t bt = i >> 7;  // rb * nsteps + t
    const int t = (int)(bt % (size_t)nsteps);
    const long long rb = (long long)(bt / (size_t)nsteps);
    const long long r = 16 * rb + (lane & 15);
    const int k0 = 128 * t + 64 * h + 16 * (lane >> 4);
    u32x4 v{0, 0, 0, 0};
    if (r < R && k0 < K) v = load16(W8 + (size_t)r * (size_t)K + k0);  // K % 16 == 0
    *reinterpret_cast<u32x4*>(P + i * 16) = v;
  }
}

// MXFP8 quantisation of bf16 rows [rows, K] (K % 32 == 0): one thread per
// block of 32 values along K.  Shared exponent = floor(log2 max |x|) - 8 (8 =
// the exponent of E4M3's largest normal), clamped to [-127, 127], -127 for a
// block of zeros or subnormals (NaN does not take part; an infinity counts as
// 2^128); elements x * 2^-shared (exact) rounded as e4m3_code.  Threads past
// K / 32 in a row write the zero padding of the scale row (stride ks).
__global__ __launch_bounds__(256) void quantize_mx_kernel(const uint16_t* __restrict__ X,
                                                          uint8_t* __restrict__ Q,
                                                          uint8_t* __restrict__ S, int rows,
                                                          int K, int ks) {
  const size_t total = (size_t)rows * ks;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (size_t)gridDim.x * blockDim.x) {
    const size_t r = t / ks;
    const int b = (int)(t % ks);
    if (b >= K / 32) {
      S[t] = 0;
      continue;
    }
    const uint16_t* x = X + r * K + 32 * b;
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = load16(x + 8 * i);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = __builtin_fabsf(bf16_to_float((uint16_t)(v[i][j] & 0xffffu)));
        const float hi = __builtin_fabsf(bf16_to_float((uint16_t)(v[i][j] >> 16)));
        if (lo > amax) amax = lo;  // comparisons with NaN are false: NaN is skipped
        if (hi > amax) amax = hi;
      }
    const int ef = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xffu);
    int shared = ef == 0 ? -127 : ef - 127 - 8;
    shared = shared < -127 ? -127 : (shared > 127 ? 127 : shared);
    S[t] = (uint8_t)(shared + 127);
    u32x4 o[2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = __builtin_ldexpf(bf16_to_float((uint16_t)(v[i][j] & 0xffffu)), -shared);
        const float hi = __builtin_ldexpf(bf16_to_float((uint16_t)(v[i][j] >> 16)), -shared);
        const uint32_t pair = e4m3_code(lo) | (e4m3_code(hi) << 8);
        const int e = 4 * i + j;  // element pair e: bytes 2e, 2e+1 of the 32
        if (e % 2 == 0)
          o[e / 8][(e % 8) / 2] = pair;
        else
          o[e / 8][(e % 8) / 2] |= pair << 16;
      }
    *reinterpret_cast<u32x4*>(Q + r * K + 32 * b) = o[0];
    *reinterpret_cast<u32x4*>(Q + r * K + 32 * b + 16) = o[1];
  }
}

// bf16 W1, W2 [K, N] -> Wt [2N, K]: Wt[2n + p, k] = Wp[k, n]; a thread writes
// one 16-byte run (8 k) of one row, neighbouring threads neighbouring rows.
__global__ __launch_bounds__(256) void pack_kmajor_kernel(const uint16_t* __restrict__ W1,
                                                          const uint16_t* __restrict__ W2,
                                                          uint16_t* __restrict__ Wt, int N,
                                                          int K) {
  const size_t rows = 2 * (size_t)N, runs = rows * (size_t)(K / 8);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < runs;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i % rows, c = i / rows;
    const int n = (int)(r >> 1);
    const uint16_t* src = ((r & 1) ? W2 : W1) + c * 8 * (size_t)N + n;
    uint32_t d[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      d[t] = (uint32_t)src[(size_t)(2 * t) * N] | ((uint32_t)src[(size_t)(2 * t + 1) * N] << 16);
    *reinterpret_cast<u32x4*>(Wt + r * (size_t)K + c * 8) = u32x4{d[0], d[1], d[2], d[3]};
  }
}

// bf16 -> E4M3 codes of fp32(x * inv_scale); 16 elements (32 B in, 16 B out)
// per thread per iteration, grid-stride.
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ X,
                                                       uint8_t* __restrict__ Q, size_t n16,
                                                       float inv_scale) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x) {
    const u32x4 lo = load16(X + i * 16);
    const u32x4 hi = load16(X + i * 16 + 8);
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32x4& s = w < 2 ? lo : hi;
      const uint32_t d0 = s[(2 * w) & 3], d1 = s[(2 * w + 1) & 3];
      const uint32_t c0 = e4m3_code(bf16_to_float((uint16_t)(d0 & 0xffffu)) * inv_scale);
      const uint32_t c1 = e4m3_code(bf16_to_float((uint16_t)(d0 >> 16)) * inv_scale);
      const uint32_t c2 = e4m3_code(bf16_to_float((uint16_t)(d1 & 0xffffu)) * inv_scale);
      const uint32_t c3 = e4m3_code(bf16_to_float((uint16_t)(d1 >> 16)) * inv_scale);
      o[w] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    *reinterpret_cast<u32x4*>(Q + i * 16) = o;
  }
}

// W8[2n + p, k] = Wp[k, n] (p = 0: W1, 1: W2), E4M3 bytes.  A thread writes
// one 16-byte run of k of one W8 row; neighbouring threads take neighbouring
// rows, so the 16 byte loads of a wave read consecutive columns.
__global__ __launch_bounds__(256) void pack_f8_kernel(const uint8_t* __restrict__ W1,
                                                      const uint8_t* __restrict__ W2,
                                                      uint8_t* __restrict__ W8, int N, int K) {
  const size_t rows = 2 * (size_t)N, runs = rows * (size_t)(K / 16);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < runs;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i % rows, c = i / rows;
    const int n = (int)(r >> 1);
    const uint8_t* src = ((r & 1) ? W2 : W1) + c * 16 * (size_t)N + n;
    uint32_t d[4] = {0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < 16; ++t) d[t >> 2] |= (uint32_t)src[(size_t)t * N] << (8 * (t & 3));
    *reinterpret_cast<u32x4*>(W8 + r * (size_t)K + c * 16) = u32x4{d[0], d[1], d[2], d[3]};
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

// Fragment-ordered W_fused from W1, W2 [K, N] (layout in front of
// packed_kernel): a thread writes one 16-byte run, the 8 consecutive k of
// W_fused column j = 128 s + 8 l + c (Gate column j/2 of W1 for even j, Up
// column j/2 of W2 for odd j), zeros outside [K, 2N].  Done once per weight
// set; the 2-byte gathers are not on any hot path.
__global__ __launch_bounds__(256) void pack_frag_kernel(const uint16_t* __restrict__ W1,
                                                        const uint16_t* __restrict__ W2,
                                                        uint16_t* __restrict__ P, int N, int K,
                                                        size_t nruns) {
  const int nsteps = (K + 31) / 32;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nruns;
       i += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63);
    const int c = (int)((i >> 6) & 7);
    const size_t st = i >> 9;  // s * nsteps + t
    const int t = (int)(st % (size_t)nsteps);
    const long long s = (long long)(st / (size_t)nsteps);
    const long long j = 128 * s + 8 * (lane & 15) + c;  // W_fused column
    const int k0 = 32 * t + 8 * (lane >> 4);
    const uint16_t* src = (j & 1) ? W2 : W1;
    const long long n = j >> 1;
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = (n < N && k0 + e < K) ? src[(size_t)(k0 + e) * (size_t)N + (size_t)n] : 0;
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = (uint32_t)v[2 * q] | ((uint32_t)v[2 * q + 1] << 16);
    *reinterpret_cast<u32x4*>(P + i * 8) = o;
  }
}

// ============================================================================
// Configuration list and launchers
// ============================================================================
// Tile rows per band of the launch order (tile_of): bands of 4 tile rows beat
// 2, 8, 16 and 64 on the 1.5B, 7B-prefill and 72B shapes (cold operands; 4 %
// faster than 8 on the 1.5B shape, 0.5-1 % on the other two).
constexpr int kGroupM = 4;

// ---- launches ------------------------------------------------------------------
// Every launch goes through hipLaunchKernel, whose return value is the status
// of that launch alone: an error that an earlier call left pending on the
// calling thread is neither reported as this launch's nor cleared.
template <typename... P, typename... Args>
static hipError_t launch_kernel(void (*k)(P...), dim3 grid, dim3 block, size_t shm,
                                hipStream_t stream, Args... args) {
  static_assert(sizeof...(P) == sizeof...(Args), "kernel argument count");
  std::tuple<std::decay_t<P>...> vals(static_cast<std::decay_t<P>>(args)...);
  return std::apply(
      [&](auto&... v) {
        void* argv[] = {static_cast<void*>(&v)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, shm, stream);
      },
      vals);
}

template <int MODE, int BM, int BNW, int BK, int STAGES, int WGM, int WGN>
static hipError_t launch_tiled(const LaunchArgs& a) {
  using C = Tiled<MODE, BM, BNW, BK, STAGES, WGM, WGN>;
  const int ntm = (a.M + BM - 1) / BM, ntn = (a.N + C::BNY - 1) / C::BNY;
  const long long nwg = (long long)ntm * ntn;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  int group_m = a.group_m > 0 ? a.group_m : kGroupM;
  if (group_m > ntm) group_m = ntm;
  return launch_kernel((tiled_kernel<MODE, BM, BNW, BK, STAGES, WGM, WGN>), dim3((unsigned)nwg),
                     dim3(C::kThreads), 0, a.stream, a.A, a.W1, a.W2, a.Y, a.M, a.N, a.K,
                     a.ldw, a.ldy, group_m);
}

// Split-tail launch: whole rounds of big tiles plus, when the last round is at
// most a quarter full, its tiles as quarter tiles; otherwise the plain kernel.
template <int MODE, int BM, int BNW, int BK, int STAGES, int WGM, int WGN, int SWGM, int SWGN>
static hipError_t launch_tiled_split(const LaunchArgs& a) {
  using C = Tiled<MODE, BM, BNW, BK, STAGES, WGM, WGN>;
  const int ntm = (a.M + BM - 1) / BM, ntn = (a.N + C::BNY - 1) / C::BNY;
  const long long nt = (long long)ntm * ntn;
  if (nt <= 0) return hipSuccess;
  if (4 * nt > 0x7fffffffLL) return hipErrorInvalidValue;
  const long long slots = a.cu_count > 0 ? a.cu_count : 256;  // one big workgroup per CU
  const long long n_big = nt / slots * slots, tail = nt - n_big;
  if (tail == 0 || 4 * tail > slots)
    return launch_tiled<MODE, BM, BNW, BK, STAGES, WGM, WGN>(a);
  int group_m = a.group_m > 0 ? a.group_m : kGroupM;
  if (group_m > ntm) group_m = ntm;
  return launch_kernel((tiled_split_kernel<MODE, BM, BNW, BK, STAGES, WGM, WGN, SWGM, SWGN>),
                     dim3((unsigned)(n_big + 4 * tail)), dim3(C::kThreads), 0, a.stream, a.A,
                     a.W1, a.W2, a.Y, a.M, a.N, a.K, a.ldw, a.ldy, group_m, (int)n_big);
}

// Persistent launch: one workgroup per CU over whole rounds of big tiles, the
// last round as quarter tiles when it is at most a quarter full.  Needs K a
// positive multiple of BK * STAGES and at least two tiles per CU; other shapes
// take the split-tail launch of the same tiles.
template <int MODE, int BM, int BNW, int BK, int STAGES, int WGM, int WGN, int SWGM, int SWGN>
static hipError_t launch_tiled_persist(const LaunchArgs& a) {
  using C = Tiled<MODE, BM, BNW, BK, STAGES, WGM, WGN>;
  const int ntm = (a.M + BM - 1) / BM, ntn = (a.N + C::BNY - 1) / C::BNY;
  const long long nt = (long long)ntm * ntn;
  const long long slots = a.cu_count > 0 ? a.cu_count : 256;  // one workgroup per CU
  if (a.K <= 0 || a.K % (BK * STAGES) != 0 || nt < 2 * slots || 4 * nt > 0x7fffffffLL)
    return launch_tiled_split<MODE, BM, BNW, BK, STAGES, WGM, WGN, SWGM, SWGN>(a);
  long long n_big = nt / slots * slots, tail = nt - n_big;
  if (tail == 0 || 4 * tail > slots) n_big = nt, tail = 0;
  int group_m = a.group_m > 0 ? a.group_m : kGroupM;
  if (group_m > ntm) group_m = ntm;
  return launch_kernel((tiled_persist_kernel<MODE, BM, BNW, BK, STAGES, WGM, WGN, SWGM, SWGN>),
                       dim3((unsigned)slots), dim3(C::kThreads), 0, a.stream, a.A, a.W1, a.Y,
                       a.M, a.N, a.K, a.ldw, a.ldy, group_m, (int)n_big, (int)(4 * tail));
}

template <int MODE, int MT, int NW>
static hipError_t launch_skinny(const LaunchArgs& a) {
  using C = Skinny<MODE, MT, NW>;
  const long long nslab = (a.N + C::SLAB_Y - 1) / C::SLAB_Y;
  const long long nmb = (a.M + MT * 16 - 1) / (MT * 16);
  if (nslab <= 0 || nmb <= 0) return hipSuccess;
  if (nslab > 0x7fffffffLL || nmb > 65535) return hipErrorInvalidValue;
  return launch_kernel((skinny_kernel<MODE, MT, NW>), dim3((unsigned)nslab, (unsigned)nmb),
                     dim3(C::kThreads), 0, a.stream, a.A, a.W1, a.W2, a.Y, a.M, a.N, a.K);
}

template <int MT, int NW, int CH>
static hipError_t launch_packed(const LaunchArgs& a) {
  using C = Packed<MT, NW, CH>;
  const long long nunit = packed_slabs(a.N) * C::PARTS;
  const long long nmb = (a.M + MT * 16 - 1) / (MT * 16);
  if (nunit <= 0 || nmb <= 0) return hipSuccess;
  if (nunit > 0x7fffffffLL || nmb > 65535) return hipErrorInvalidValue;
  return launch_kernel((packed_kernel<MT, NW, CH>), dim3((unsigned)nunit, (unsigned)nmb),
                     dim3(C::kThreads), 0, a.stream, a.A, a.W1, a.Y, a.M, a.N, a.K);
}

template <int NW>
static hipError_t launch_packed_mixed(const LaunchArgs& a) {
  const long long slabs = packed_slabs(a.N);
  const long long nmb = (a.M + 15) / 16;
  if (slabs <= 0 || nmb <= 0) return hipSuccess;
  const long long cus = a.cu_count > 0 ? a.cu_count : 256;
  const long long nwhole = slabs / cus * cus;
  const long long nunit = nwhole + (slabs - nwhole) * 4;
  if (nunit > 0x7fffffffLL || nmb > 65535) return hipErrorInvalidValue;
  return launch_kernel((packed_mixed_kernel<NW>), dim3((unsigned)nunit, (unsigned)nmb),
                       dim3(64 * NW), 0, a.stream, a.A, a.W1, a.Y, a.M, a.N, a.K, (int)nwhole);
}

template <int NW, int CH>
static hipError_t launch_packed_splitk(const LaunchArgs& a) {
  using C = Packed<1, NW, CH>;
  const long long slabs = packed_slabs(a.N);
  const long long nunit = slabs * C::PARTS * (long long)a.ksplit;
  if (a.M <= 0 || nunit <= 0) return hipSuccess;
  if (a.ksplit < 1 || a.M > 16 || nunit > 0x7fffffffLL || !a.ws) return hipErrorInvalidValue;
  uint32_t* counters = static_cast<uint32_t*>(a.ws);
  f32x4* partials =
      reinterpret_cast<f32x4*>(static_cast<uint8_t*>(a.ws) + splitk_counter_bytes(slabs));
  return launch_kernel((packed_splitk_kernel<NW, CH>), dim3((unsigned)nunit), dim3(C::kThreads),
                       0, a.stream, a.A, a.W1, a.Y, a.M, a.N, a.K, a.ksplit, counters, partials);
}

template <int MODE, int BM, int BNW, int STAGES, int WGM, int WGN>
static hipError_t launch_f8(const LaunchArgs& a) {
  using C = F8Tiled<MODE, BM, BNW, STAGES, WGM, WGN>;
  const int ntm = (a.M + BM - 1) / BM, ntn = (a.N + C::BNY - 1) / C::BNY;
  const long long nwg = (long long)ntm * ntn;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  int group_m = a.group_m > 0 ? a.group_m : kGroupM;
  if (group_m > ntm) group_m = ntm;
  return launch_kernel((f8_kernel<MODE, BM, BNW, STAGES, WGM, WGN>), dim3((unsigned)nwg),
                     dim3(C::kThreads), 0, a.stream, (const uint8_t*)a.A,
                     (const uint8_t*)a.W1, a.Y, a.M, a.N, a.K, a.scale_g, a.scale_u, a.SA, a.SW,
                     a.ks, group_m);
}

template <int MODE, int BM, int BNW, int STAGES, int WGM, int WGN, int SWGM, int SWGN>
static hipError_t launch_f8_split(const LaunchArgs& a) {
  using C = F8Tiled<MODE, BM, BNW, STAGES, WGM, WGN>;
  const int ntm = (a.M + BM - 1) / BM, ntn = (a.N + C::BNY - 1) / C::BNY;
  const long long nt = (long long)ntm * ntn;
  if (nt <= 0) return hipSuccess;
  if (4 * nt > 0x7fffffffLL) return hipErrorInvalidValue;
  const long long slots = a.cu_count > 0 ? a.cu_count : 256;
  const long long n_big = nt / slots * slots, tail = nt - n_big;
  if (tail == 0 || 4 * tail > slots) return launch_f8<MODE, BM, BNW, STAGES, WGM, WGN>(a);
  int group_m = a.group_m > 0 ? a.group_m : kGroupM;
  if (group_m > ntm) group_m = ntm;
  return launch_kernel((f8_split_kernel<MODE, BM, BNW, STAGES, WGM, WGN, SWGM, SWGN>),
                     dim3((unsigned)(n_big + 4 * tail)), dim3(C::kThreads), 0, a.stream,
                     (const uint8_t*)a.A, (const uint8_t*)a.W1, a.Y, a.M, a.N, a.K, a.scale_g,
                     a.scale_u, a.SA, a.SW, a.ks, group_m, (int)n_big);
}

template <int MT, int NB, int NW>
static hipError_t launch_f8_skinny(const LaunchArgs& a) {
  using C = F8Skinny<MT, NB, NW>;
  const long long nslab = (2LL * a.N + C::SLAB_W - 1) / C::SLAB_W;
  const long long nmb = (a.M + MT * 16 - 1) / (MT * 16);
  if (nslab <= 0 || nmb <= 0) return hipSuccess;
  if (nslab > 0x7fffffffLL || nmb > 65535) return hipErrorInvalidValue;
  return launch_kernel((f8_skinny_kernel<MT, NB, NW>), dim3((unsigned)nslab, (unsigned)nmb),
                     dim3(C::kThreads), 0, a.stream, (const uint8_t*)a.A, (const uint8_t*)a.W1,
                     a.Y, a.M, a.N, a.K, a.scale_g, a.scale_u);
}

template <int MT, int NB, int NW>
static hipError_t launch_f8_packed(const LaunchArgs& a) {
  using C = F8Packed<MT, NB, NW>;
  const long long nunit = (2LL * a.N + C::SLAB_W - 1) / C::SLAB_W;
  const long long nmb = (a.M + MT * 16 - 1) / (MT * 16);
  if (nunit <= 0 || nmb <= 0) return hipSuccess;
  if (nunit > 0x7fffffffLL || nmb > 65535) return hipErrorInvalidValue;
  return launch_kernel((f8_packed_kernel<MT, NB, NW>), dim3((unsigned)nunit, (unsigned)nmb),
                     dim3(C::kThreads), 0, a.stream, (const uint8_t*)a.A, (const uint8_t*)a.W1,
                     a.Y, a.M, a.N, a.K, a.scale_g, a.scale_u);
}

#define F8_PACKED(mt, nb, nw)                                                              \
  {VAR_F8_PACKED, 1, (mt) * 16, F8Packed<mt, nb, nw>::SLAB_Y, 128, nw, nw,                  \
   F8Packed<mt, nb, nw>::LDS_BYTES, &launch_f8_packed<mt, nb, nw>}
template <int NB, int NW>
static hipError_t launch_mx_packed(const LaunchArgs& a) {
  using C = MxPacked<NB, NW>;
  const long long nunit = (2LL * a.N + C::SLAB_W - 1) / C::SLAB_W;
  const long long nmb = (a.M + 31) / 32;
  if (nunit <= 0 || nmb <= 0) return hipSuccess;
  if (nunit > 0x7fffffffLL || nmb > 65535) return hipErrorInvalidValue;
  return launch_kernel((mx_packed_kernel<NB, NW>), dim3((unsigned)nunit, (unsigned)nmb),
                     dim3(C::kThreads), 0,
                     a.stream, (const uint8_t*)a.A, a.SA, (const uint8_t*)a.W1, a.SW, a.Y, a.M,
                     a.N, a.K, a.ks);
}

#define MX_PACKED(nb, nw)                                                                  \
  {VAR_MX_PACKED, 1, 32, MxPacked<nb, nw>::SLAB_Y, 64, nw, nw, MxPacked<nb, nw>::LDS_BYTES,    \
   &launch_mx_packed<nb, nw>}
#define F8_SKINNY(mt, nb, nw)                                                              \
  {VAR_F8, 1, (mt) * 16, F8Skinny<mt, nb, nw>::SLAB_Y, 128, nw, nw,                         \
   F8Skinny<mt, nb, nw>::LDS_BYTES, &launch_f8_skinny<mt, nb, nw>}
#define F8(mode, v, bm, bnw, st, wgm, wgn)                                                 \
  {v, 0, bm, F8Tiled<mode, bm, bnw, st, wgm, wgn>::BNY, 64, (wgm) * (wgn), 1,              \
   F8Tiled<mode, bm, bnw, st, wgm, wgn>::LDS_BYTES, &launch_f8<mode, bm, bnw, st, wgm, wgn>}
#define F8_SPLIT(mode, v, bm, bnw, st, wgm, wgn, swgm, swgn)                               \
  {v, 0, bm, F8Tiled<mode, bm, bnw, st, wgm, wgn>::BNY, 64, (wgm) * (wgn), 1,              \
   F8Tiled<mode, bm, bnw, st, wgm, wgn>::LDS_BYTES,                                        \
   &launch_f8_split<mode, bm, bnw, st, wgm, wgn, swgm, swgn>, 4}
#define TILED(mode, v, bm, bnw, bk, st, wgm, wgn)                                          \
  {v, 0, bm, Tiled<mode, bm, bnw, bk, st, wgm, wgn>::BNY, bk, (wgm) * (wgn), 1,             \
   Tiled<mode, bm, bnw, bk, st, wgm, wgn>::LDS_BYTES, &launch_tiled<mode, bm, bnw, bk, st, wgm, wgn>}
#define TILED_SPLIT(mode, v, bm, bnw, bk, st, wgm, wgn, swgm, swgn)                          \
  {v, 0, bm, Tiled<mode, bm, bnw, bk, st, wgm, wgn>::BNY, bk, (wgm) * (wgn), 1,             \
   Tiled<mode, bm, bnw, bk, st, wgm, wgn>::LDS_BYTES,                                       \
   &launch_tiled_split<mode, bm, bnw, bk, st, wgm, wgn, swgm, swgn>, 4}
#define TILED_PERSIST(mode, v, bm, bnw, bk, st, wgm, wgn, swgm, swgn)                        \
  {v, 2, bm, Tiled<mode, bm, bnw, bk, st, wgm, wgn>::BNY, bk, (wgm) * (wgn), 1,             \
   Persist<mode, bm, bnw, bk, st, wgm, wgn>::LDS_BYTES,                                     \
   &launch_tiled_persist<mode, bm, bnw, bk, st, wgm, wgn, swgm, swgn>, 4}
#define PACKED_SPLITK(nw, ch)                                                              \
  {VAR_PACKED_SPLITK, 3, 16, Packed<1, nw, ch>::COLS_Y, 32, nw, nw, Packed<1, nw, ch>::LDS_BYTES, \
   &launch_packed_splitk<nw, ch>}
#define PACKED(mt, nw, ch)                                                                 \
  {VAR_PACKED, 1, (mt) * 16, Packed<mt, nw, ch>::COLS_Y, 32, nw, nw,                          \
   Packed<mt, nw, ch>::LDS_BYTES, &launch_packed<mt, nw, ch>}
#define SKINNY(mode, v, mt, nw)                                                            \
  {v, 1, (mt) * 16, Skinny<mode, mt, nw>::SLAB_Y, 32, nw, nw, Skinny<mode, mt, nw>::LDS_BYTES, \
   &launch_skinny<mode, mt, nw>}

static const KernelConfig kConfigs[] = {
    // ---- interleave (Kernel-2 family) --------------------------------------
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 256, 256, 32, 4, 2, 2),  // 0
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 128, 256, 32, 4, 2, 2),  // 1
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 128, 128, 32, 4, 2, 2),  // 2
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 64, 128, 32, 4, 2, 2),   // 3
    SKINNY(MODE_INTERLEAVE, VAR_INTERLEAVE, 1, 8),                  // 4
    SKINNY(MODE_INTERLEAVE, VAR_INTERLEAVE, 2, 8),                  // 5
    SKINNY(MODE_INTERLEAVE, VAR_INTERLEAVE, 4, 4),                  // 6
    // ---- sync (Kernel-1 family) --------------------------------------------
    TILED(MODE_SYNC, VAR_SYNC, 256, 128, 32, 4, 2, 2),              // 7
    TILED(MODE_SYNC, VAR_SYNC, 128, 128, 32, 4, 2, 2),              // 8
    TILED(MODE_SYNC, VAR_SYNC, 128, 64, 32, 4, 2, 2),               // 9
    TILED(MODE_SYNC, VAR_SYNC, 64, 64, 32, 4, 2, 2),                // 10
    SKINNY(MODE_SYNC, VAR_SYNC, 1, 8),                              // 11
    SKINNY(MODE_SYNC, VAR_SYNC, 2, 8),                              // 12
    SKINNY(MODE_SYNC, VAR_SYNC, 4, 4),                              // 13
    // ---- plain GEMM for the unfused baseline -------------------------------
    TILED(MODE_GEMM, VAR_GEMM, 256, 256, 32, 4, 2, 2),              // 14
    TILED(MODE_GEMM, VAR_GEMM, 256, 128, 32, 4, 2, 2),              // 15
    TILED(MODE_GEMM, VAR_GEMM, 128, 128, 32, 4, 2, 2),              // 16
    TILED(MODE_GEMM, VAR_GEMM, 64, 64, 32, 4, 2, 2),                // 17
    SKINNY(MODE_GEMM, VAR_GEMM, 1, 8),                              // 18
    SKINNY(MODE_GEMM, VAR_GEMM, 2, 8),                              // 19
    SKINNY(MODE_GEMM, VAR_GEMM, 4, 4),                              // 20
    // ---- tiles sized for wave quantisation on 256 CUs ----------------------
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 256, 192, 32, 4, 2, 2),  // 21
    TILED(MODE_GEMM, VAR_GEMM, 256, 192, 32, 4, 2, 2),              // 22
    // ---- small M with four waves per workgroup (two workgroups per CU) -----
    SKINNY(MODE_INTERLEAVE, VAR_INTERLEAVE, 1, 4),                  // 23
    SKINNY(MODE_INTERLEAVE, VAR_INTERLEAVE, 2, 4),                  // 24
    SKINNY(MODE_SYNC, VAR_SYNC, 1, 4),                              // 25
    SKINNY(MODE_GEMM, VAR_GEMM, 1, 4),                              // 26
    // ---- small tiles with deep stage rings (latency-bound shapes) ----------
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 64, 128, 32, 8, 2, 2),   // 27
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 128, 128, 32, 8, 2, 2),  // 28
    TILED(MODE_SYNC, VAR_SYNC, 64, 64, 32, 8, 2, 2),                // 29
    TILED(MODE_GEMM, VAR_GEMM, 64, 64, 32, 8, 2, 2),                // 30
    // ---- eight waves per workgroup: two per SIMD hide each other's stalls ----
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 256, 256, 32, 4, 2, 4),  // 31
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 256, 256, 32, 4, 4, 2),  // 32
    TILED(MODE_GEMM, VAR_GEMM, 256, 256, 32, 4, 2, 4),              // 33
    TILED(MODE_SYNC, VAR_SYNC, 256, 128, 32, 4, 2, 4),              // 34
    TILED(MODE_INTERLEAVE, VAR_INTERLEAVE, 256, 192, 32, 4, 4, 2),  // 35
    // ---- the split 256-row tiles on one persistent workgroup per CU, the
    //      next tile's loads running under each tile's last steps ----------
    TILED_PERSIST(MODE_INTERLEAVE, VAR_INTERLEAVE, 256, 256, 32, 4, 4, 2, 2, 4),  // 36
    TILED_PERSIST(MODE_GEMM, VAR_GEMM, 256, 256, 32, 4, 4, 2, 2, 4),              // 37
    // ---- eight waves as 4 x 2 (64-row wave tiles) for the other modes -----
    TILED(MODE_GEMM, VAR_GEMM, 256, 256, 32, 4, 4, 2),              // 38
    TILED(MODE_SYNC, VAR_SYNC, 256, 128, 32, 4, 4, 2),              // 39
    // ---- 256 x 256 tiles whose partial last round runs as quarter tiles ----
    TILED_SPLIT(MODE_INTERLEAVE, VAR_INTERLEAVE, 256, 256, 32, 4, 4, 2, 2, 4),  // 40
    TILED_SPLIT(MODE_GEMM, VAR_GEMM, 256, 256, 32, 4, 4, 2, 2, 4),              // 41
    TILED_SPLIT(MODE_SYNC, VAR_SYNC, 256, 128, 32, 4, 4, 2, 4, 2),              // 42
    // ---- FP8 (E4M3) inputs, k-contiguous paired weights ----------------------
    F8_SPLIT(MODE_INTERLEAVE, VAR_F8, 256, 256, 4, 4, 2, 2, 4),     // 43
    F8(MODE_INTERLEAVE, VAR_F8, 256, 256, 4, 4, 2),                 // 44
    F8(MODE_INTERLEAVE, VAR_F8, 128, 256, 4, 2, 2),                 // 45
    F8(MODE_INTERLEAVE, VAR_F8, 64, 128, 4, 2, 2),                  // 46
    F8(MODE_INTERLEAVE, VAR_F8, 64, 128, 8, 2, 2),                  // 47
    F8_SKINNY(1, 8, 4),                                             // 48
    F8_SKINNY(1, 4, 4),                                             // 49
    F8_SKINNY(2, 8, 4),                                             // 50
    F8_SKINNY(4, 4, 4),                                             // 51
    // one wave per workgroup, each streaming 32 W8 rows over the whole K
    F8_SKINNY(1, 2, 1),                                             // 52
    // ---- FP8 sync (Kernel-1 order) on the same W8 ----------------------------
    F8_SPLIT(MODE_SYNC, VAR_F8_SYNC, 256, 128, 4, 4, 2, 4, 2),      // 53
    F8(MODE_SYNC, VAR_F8_SYNC, 128, 128, 4, 2, 2),                  // 54
    F8(MODE_SYNC, VAR_F8_SYNC, 64, 64, 4, 2, 2),                    // 55
    // ---- MXFP8 (E8M0 block scales applied by the MFMA) ---------------------
    F8_SPLIT(MODE_MX, VAR_MX, 256, 256, 4, 4, 2, 2, 4),             // 56
    F8(MODE_MX, VAR_MX, 64, 128, 4, 2, 2),                          // 57
    // ---- fragment-ordered W_fused (split-K streaming, no transposition) ----
    PACKED(1, 4, 8),                                                // 58
    PACKED(1, 8, 8),                                                // 59
    PACKED(2, 4, 8),                                                // 60
    PACKED(2, 8, 8),                                                // 61
    PACKED(4, 4, 8),                                                // 62
    // a slab split over 4 or 2 workgroups (even load over the CUs)
    PACKED(1, 4, 2),                                                // 63
    PACKED(1, 8, 2),                                                // 64
    PACKED(1, 4, 4),                                                // 65
    PACKED(1, 8, 4),                                                // 66
    PACKED(2, 4, 2),                                                // 67
    PACKED(4, 4, 2),                                                // 68
    PACKED(2, 4, 4),                                                // 69
    // ---- FP8 on fragment-ordered W8 (streaming) ------------------------------
    F8_PACKED(1, 2, 1),                                             // 70
    F8_PACKED(1, 1, 1),                                             // 71
    F8_PACKED(1, 2, 2),                                             // 72
    F8_PACKED(1, 4, 1),                                             // 73
    F8_PACKED(1, 4, 2),                                             // 74
    F8_PACKED(2, 2, 1),                                             // 75
    F8_PACKED(4, 2, 1),                                             // 76
    // ---- MXFP8 on fragment-ordered W8 (streaming, 32x32x64 scaled MFMA) -----
    MX_PACKED(1, 1),                                                // 77
    MX_PACKED(2, 1),                                                // 78
    MX_PACKED(4, 1),                                                // 79
    MX_PACKED(1, 2),                                                // 80
    MX_PACKED(1, 4),                                                // 81
    // ---- MXFP8 in the sync (Kernel-1) order on the same W8 ---------------
    F8_SPLIT(MODE_MX_SYNC, VAR_MX_SYNC, 256, 128, 4, 4, 2, 4, 2),   // 82
    F8(MODE_MX_SYNC, VAR_MX_SYNC, 128, 128, 4, 2, 2),               // 83
    F8(MODE_MX_SYNC, VAR_MX_SYNC, 64, 64, 4, 2, 2),                 // 84
    // ---- fragment-ordered W_fused streaming with K split over workgroups ----
    PACKED_SPLITK(4, 8),                                            // 85
    PACKED_SPLITK(4, 4),                                            // 86
    PACKED_SPLITK(4, 2),                                            // 87
    // ---- fragment-ordered W_fused: whole slabs, then quarter slabs --------
    {VAR_PACKED, 1, 16, Packed<1, 8, 8>::COLS_Y, 32, 8, 8, Packed<1, 8, 8>::LDS_BYTES,
     &launch_packed_mixed<8>},                                      // 88
    // ---- sync family on W1 and W2 as stored: Gate and Up wave groups share
    //      each A k-tile, SiLU(Gate) handed over through LDS ----------------
    TILED_SPLIT(MODE_PAIR, VAR_SYNC, 256, 256, 32, 4, 4, 2, 4, 2),  // 89
    TILED(MODE_PAIR, VAR_SYNC, 128, 256, 32, 4, 2, 2),              // 90
    TILED(MODE_PAIR, VAR_SYNC, 128, 128, 32, 4, 2, 2),              // 91
    TILED(MODE_PAIR, VAR_SYNC, 64, 128, 32, 4, 2, 2),               // 92
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
  return launch_kernel(gate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, G, U, Y, n8);
}

hipError_t launch_quantize_f8(const uint16_t* X, uint8_t* Q, size_t n, float inv_scale,
                              hipStream_t stream, int cu_count) {
  const size_t n16 = n / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  const size_t cap = (size_t)(cu_count > 0 ? cu_count : 256) * 8;
  if (blocks > cap) blocks = cap;
  return launch_kernel(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, X, Q, n16,
                     inv_scale);
}

hipError_t launch_quantize_mx(const uint16_t* X, uint8_t* Q, uint8_t* S, int rows, int K, int ks,
                              hipStream_t stream, int cu_count) {
  const size_t total = (size_t)rows * ks;
  if (total == 0) return hipSuccess;
  size_t blocks = (total + 255) / 256;
  const size_t cap = (size_t)(cu_count > 0 ? cu_count : 256) * 8;
  if (blocks > cap) blocks = cap;
  return launch_kernel(quantize_mx_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, X, Q, S,
                     rows, K, ks);
}

hipError_t launch_pack_kmajor(const uint16_t* W1, const uint16_t* W2, uint16_t* Wt, int N, int K,
                              hipStream_t stream, int cu_count) {
  const size_t runs = 2 * (size_t)N * (size_t)(K / 8);
  if (runs == 0) return hipSuccess;
  size_t blocks = (runs + 255) / 256;
  const size_t cap = (size_t)(cu_count > 0 ? cu_count : 256) * 8;
  if (blocks > cap) blocks = cap;
  return launch_kernel(pack_kmajor_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W1, W2, Wt,
                     N, K);
}

hipError_t launch_pack_f8(const uint8_t* W1, const uint8_t* W2, uint8_t* W8, int N, int K,
                          hipStream_t stream, int cu_count) {
  const size_t runs = 2 * (size_t)N * (size_t)(K / 16);
  if (runs == 0) return hipSuccess;
  size_t blocks = (runs + 255) / 256;
  const size_t cap = (size_t)(cu_count > 0 ? cu_count : 256) * 8;
  if (blocks > cap) blocks = cap;
  return launch_kernel(pack_f8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W1, W2, W8, N,
                     K);
}

hipError_t launch_pack_mx_frag(const uint8_t* W8, uint8_t* P, int R, int K, hipStream_t stream,
                              int cu_count) {
  const size_t nchunks = (size_t)((R + 31) / 32) * (size_t)(K / 64) * 128;
  if (nchunks == 0) return hipSuccess;
  size_t blocks = (nchunks + 255) / 256;
  const size_t cap = (size_t)(cu_count > 0 ? cu_count : 256) * 8;
  if (blocks > cap) blocks = cap;
  return launch_kernel(pack_mx_frag_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W8, P, R,
                     K, nchunks);
}

hipError_t launch_pack_f8_frag(const uint8_t* W8, uint8_t* P, int R, int K, hipStream_t stream,
                              int cu_count) {
  const size_t nchunks = (size_t)((R + 15) / 16) * (size_t)((K + 127) / 128) * 128;
  if (nchunks == 0) return hipSuccess;
  size_t blocks = (nchunks + 255) / 256;
  const size_t cap = (size_t)(cu_count > 0 ? cu_count : 256) * 8;
  if (blocks > cap) blocks = cap;
  return launch_kernel(pack_f8_frag_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W8, P, R,
                     K, nchunks);
}

hipError_t launch_pack_frag(const uint16_t* W1, const uint16_t* W2, uint16_t* P, int N, int K,
                           hipStream_t stream, int cu_count) {
  const size_t nruns = (size_t)packed_slabs(N) * (size_t)packed_steps(K) * 512;
  if (nruns == 0) return hipSuccess;
  size_t blocks = (nruns + 255) / 256;
  const size_t cap = (size_t)(cu_count > 0 ? cu_count : 256) * 8;
  if (blocks > cap) blocks = cap;
  return launch_kernel(pack_frag_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W1, W2, P,
                     N, K, nruns);
}

hipError_t launch_pack(const uint16_t* W1, const uint16_t* W2, uint16_t* WF, size_t n,
                       hipStream_t stream, int cu_count) {
  const size_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  size_t blocks = (n8 + 255) / 256;
  const size_t cap = (size_t)(cu_count > 0 ? cu_count : 256) * 8;
  if (blocks > cap) blocks = cap;
  return launch_kernel(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W1, W2, WF, n8);
}

}  // namespace swiglu
