// swiglu_table.cpp -- per-shape tile and occupancy table.
//
// The page describing the method picks its kernel by batch size: the sync
// kernel for large batches (M >= 2048), where an [M, N] grid of tiles already
// fills the machine, and the interleave kernel for small ones, where doubling
// the number of tiles raises occupancy ("Riepilogo Tecnico: Sovrapposizione
// delle Attivazioni a Livello di Tile...", §Metodologia, Kernel-1 and Kernel-2
// "Ottimizzazione"; §Contributi Chiave item 2).  Here the same decision is
// re-made for MI355X: exact entries come from measured sweeps on the
// Qwen2.5-shaped MLP workloads; every other shape takes the fallback rule, a
// choice by M measured on an M sweep (256 ... 8192) at the 1.5B K and N.
#include "swiglu_internal.h"

namespace swiglu {

namespace {

struct ShapeEntry {
  int variant;
  long long M, N, K;
  int config_id;
};

// Measured best configurations (MI355X, bf16, inputs HBM-resident).  The list
// only ever records a configuration that won its sweep, so the table cannot
// pick something slower than the fallback it replaces.
const ShapeEntry kTable[] = {
    // Qwen2.5-0.5B MLP, M=128
    {VAR_INTERLEAVE, 128, 4864, 896, 3},
    {VAR_SYNC, 128, 4864, 896, 29},
    {VAR_GEMM, 128, 4864, 896, 30},
    // Qwen2.5-1.5B MLP, M=2048
    {VAR_INTERLEAVE, 2048, 8960, 1536, 40},
    {VAR_SYNC, 2048, 8960, 1536, 42},
    {VAR_GEMM, 2048, 8960, 1536, 41},
    // Qwen2.5-7B MLP, decode M=16 and prefill M=8192
    {VAR_INTERLEAVE, 16, 18944, 3584, 23},
    {VAR_SYNC, 16, 18944, 3584, 12},
    {VAR_GEMM, 16, 18944, 3584, 18},
    {VAR_INTERLEAVE, 8192, 18944, 3584, 40},
    {VAR_SYNC, 8192, 18944, 3584, 42},
    {VAR_GEMM, 8192, 18944, 3584, 41},
    // Qwen2.5-72B MLP, M=4096
    {VAR_INTERLEAVE, 4096, 29568, 8192, 40},
    {VAR_SYNC, 4096, 29568, 8192, 42},
    {VAR_GEMM, 4096, 29568, 8192, 41},
    // one GPU's share under 8-way tensor parallelism (N / 8), where the tuner
    // beat the fallback rule by more than 3 %
    {VAR_SYNC, 8192, 2368, 3584, 8},          // 7B prefill share: 348 vs 376 us
    {VAR_INTERLEAVE, 16, 2368, 3584, 27},     // 7B decode share: 22.9 vs 23.6 us
    {VAR_GEMM, 16, 2368, 3584, 30},           // 32.1 vs 49.2 us
    {VAR_INTERLEAVE, 128, 608, 896, 5},       // 0.5B share: 7.6 vs 7.9 us
    {VAR_SYNC, 128, 608, 896, 12},            // 9.0 vs 13.6 us
    {VAR_PACKED, 128, 608, 896, 67},          // 4.6 vs 9.2 us
    // batches of 32 and 64 rows on the 72B matrices: the 128 x 256 tile beats
    // weight streaming (tuner: 156.4 vs 172.3 us at M = 32, 157.3 vs 193.3 us at
    // M = 64); FP8 split-K streaming with 32-row blocks at M = 32
    {VAR_INTERLEAVE, 32, 29568, 8192, 1},
    {VAR_INTERLEAVE, 64, 29568, 8192, 1},
    {VAR_F8, 32, 29568, 8192, 50},            // 93.1 vs 108.0 us
    {VAR_PACKED, 32, 29568, 8192, 62},        // 163.1 vs 182.6 us
    // larger batches on the 7B and 72B matrices (tuner)
    {VAR_F8, 2048, 29568, 8192, 44},          // no split tail: 879 vs 957 us
    {VAR_SYNC, 1024, 18944, 3584, 8},         // 359 vs 375 us
    {VAR_F8_SYNC, 1024, 18944, 3584, 54},     // 184 vs 196 us
    // decode-sized batches on the 0.5B and 1.5B matrices (tuner)
    {VAR_SYNC, 64, 4864, 896, 12},            // 11.4 vs 14.6 us
    {VAR_PACKED, 64, 4864, 896, 69},          // 8.3 vs 11.2 us
    {VAR_PACKED, 16, 8960, 1536, 63},         // 14.3 vs 15.1 us
    // batch sizes where tile rounds quantise against the wide-matrix rules
    // (tuner, 7B K and N): three exact 128-row tiles beat two 256-row ones at
    // M = 384 for sync and FP8; the 256 x 256 GEMM tile keeps M = 768 in one
    // round (222 tiles, 198.5 us; 256 x 192 needs 297 tiles, 327.9 us)
    {VAR_SYNC, 384, 18944, 3584, 8},          // 163.3 vs 205.9 us
    {VAR_F8, 384, 18944, 3584, 45},           // 74.8 vs 94.7 us
    {VAR_GEMM, 768, 18944, 3584, 14},         // 198.5 vs 327.9 us
    {VAR_INTERLEAVE, 384, 18944, 3584, 40},   // 130.5 vs 137.1 us (the round model says 1)
};

int find_config(int variant, int family, int bm, int bn, int waves) {
  for (int i = 0; i < config_count(); ++i) {
    const KernelConfig* c = config_at(i);
    if (c->variant == variant && c->family == family && c->bm == bm && c->bn == bn &&
        (waves == 0 || c->waves == waves))
      return i;
  }
  return -1;
}

// Estimated time of covering an M x N output with tiles of bm rows and bny
// output columns, in rounds of one workgroup per CU weighted by tile size:
// whole rounds, then a partial last round, which split configurations run as
// quarter tiles (counted as half a round when it is at most a quarter full).
// A 256-row tile costs 1.8 times a 128-row one at K = 3584 and 1.4 times from
// K = 4096 (its fixed per-tile cost is spread over a longer K loop): fitted to
// the tuner's measurements on the 7B and 72B matrices (sync, FP8 and
// interleave, M = 160 ... 1024; the 32B matrices at K = 5120 follow the 72B
// weight: M = 384 sync 307.7 vs 348.1 us, FP8 140.2 vs 163.2 us), where it
// picks the measured best or a configuration within 2 % of it; used only up
// to M = 768, the range measured for every family.
double tile_rounds(long long M, long long N, long long K, int bm, int bny, bool split,
                   long long cus) {
  const long long tiles = ((M + bm - 1) / bm) * ((N + bny - 1) / bny);
  const long long full = tiles / cus, tail = tiles % cus;
  const double last = tail == 0 ? 0.0 : ((split && 4 * tail <= cus) ? 0.5 : 1.0);
  return ((double)full + last) * (bm == 256 ? (K >= 4096 ? 1.4 : 1.8) : 1.0);
}

}  // namespace

int select_config(int variant, long long M, long long N, long long K, int cu_count) {
  for (const ShapeEntry& e : kTable)
    if (e.variant == variant && e.M == M && e.N == N && e.K == K) return e.config_id;
  // Narrow N: when the 256-row tiles (128 output columns each) would leave more
  // than half of the CUs without a tile, smaller tiles win (tuner, 1.5B share
  // under 8-way tensor parallelism, M = 2048, N = 1120: 72 big tiles; bf16
  // 25.9 vs 34.5 us interleave, 36.4 vs 48.6 us sync; FP8 15.8 vs 20.4 us;
  // MXFP8 20.6 vs 23.1 us).
  const long long cus = cu_count > 0 ? cu_count : 256;
  const bool few_big = ((M + 255) / 256) * ((N + 127) / 128) * 2 < cus;
  // Wide N (at least half a CU's worth of 256-wide W_fused column tiles, i.e.
  // N >= 16384 on 256 CUs): from M = 65 on, 256-row tiles already give every
  // CU work and their higher arithmetic intensity wins over the small tiles
  // chosen for narrower matrices (tuner, 7B and 72B K and N: M = 128 35-38 %,
  // M = 256 37 % faster in bf16; FP8 20-28 %, MXFP8 10-21 %).
  const bool wide = (2 * N + 255) / 256 * 2 >= cus;
  // Mid-width N (not wide, but 64-wide W_fused column tiles alone give every
  // CU a tile: the 1.5B and 3B matrices, not the 0.5B one): from M = 65 one
  // band of 128-row tiles already fills the chip, and the 64-row tiles' second
  // pass over W_fused costs more than their parallelism gains (tuner, 1.5B and
  // 3B, M = 80 ... 192: interleave 19-23 %, sync 9-28 %, GEMM 4-17 %).
  const bool mid = !wide && (2 * N + 63) / 64 >= cus;
  // On mid-width N from M = 129 to 160, 64-row tiles still win while all of
  // them fit in one round of four workgroups per CU (1.5B, M = 144: sync
  // 31.3 vs 34.7 us, GEMM 36.8 vs 39.6 us); past that (3B, M = 160: 1032
  // tiles) the 128 x 128 tiles do (sync 44.5 vs 61.3 us, GEMM 49.8 vs 59.5 us).
  const bool one_round64 = ((M + 63) / 64) * ((2 * N + 63) / 64) <= 4 * cus;
  // Mid-width N with a long K loop (14B: K = 5120, N = 13824): from M = 129
  // (interleave: 257) to 768 the tiles follow the wide-matrix rules, because
  // a 256-row tile's fixed cost is spread over the long loop (tuner, M = 384:
  // interleave 109.7 vs 187.2 us, sync 156.8 vs 228.7 us, FP8 70.6 vs 111.3
  // us; M = 192: FP8 sync 64.4 vs 92.3 us).
  const bool long_k = mid && K >= 4096 && M <= 768;
  // Narrower, but 64-wide W_fused column tiles still cover half of the CUs,
  // with a long K loop (72B share under 4-way tensor parallelism; not the
  // 8-way one, N = 3696, where the rules for narrow matrices stay best).
  const bool half_long_k = !wide && !mid && K >= 4096 && 2 * ((2 * N + 63) / 64) >= cus;
  // FP8 sync order (measured on the five workloads: 128 x 128 tiles won at
  // M = 2048, the split 256-row tiles at M = 4096 and 8192)
  // MXFP8: 64 x 128 tiles for small M, the split 256 x 256 tiles above
  if (variant == VAR_MX) return (M <= 64 || (M <= 192 && !wide) || few_big) ? 57 : 56;
  // MXFP8 on fragment-ordered W8: blocks of 32 W8 rows by 32-row groups of A
  // at any M; one block and one wave per workgroup (7B decode: 1184
  // workgroups, 25.6 us against 27.1 with two blocks), four blocks from 6
  // blocks per CU (72B: 79.5 us against 92.1 with one), and K split over four
  // waves below one block per CU (8-way tensor-parallel shares of 7B and 72B:
  // 8.9 and 17.6 us against 19.7 and 42.0 with one wave)
  if (variant == VAR_MX_PACKED) {
    const long long blocks = (2 * N + 31) / 32;
    return blocks >= 6 * cus ? 79 : (blocks >= cus ? 77 : 81);
  }
  if (variant == VAR_PACKED) {
    // fragment-ordered weights (measured at M = 16, 32, 48, 64 on the 0.5B,
    // 7B and 72B K and N): each CU streams at a bounded rate, so a launch
    // wants its slabs spread evenly over the CUs -- whole slabs when there
    // are at least 1.75 per CU (72B: 462), half slabs from half a slab per
    // CU (7B: 296 slabs -> 592 workgroups), quarter slabs below (0.5B: 76).
    // Above M = 16 the 32- and 64-row blocks win; above M = 64 the weights
    // are re-read once per 64 rows (a fallback, not a fast path).
    // Narrow N (under 64 slabs: one GPU's share under 8-way tensor
    // parallelism) takes 8 waves per quarter slab (tuner: +3-5 %).
    const long long slabs = packed_slabs(N);
    if (M <= 16)
      return 4 * slabs >= 7 * cus ? 58 : (2 * slabs >= cus ? 65 : (slabs >= 64 ? 63 : 64));
    return M <= 32 ? 69 : 62;
  }
  // FP8 on fragment-ordered W8: streaming by 16-row groups at any M; one
  // wave per 32 W8 rows, two waves splitting K when that leaves fewer than two
  // workgroups per CU (tuner at N = 2368 and 3696: +29 %)
  if (variant == VAR_F8_PACKED) {
    const long long units = (2 * N + 31) / 32;
    if (M <= 16) return units >= 2 * cus ? 70 : 72;
    // 33-64 rows: 32-row blocks on narrower matrices (0.5B: 5.8 vs 6.9 us)
    return (M <= 32 || !wide) ? 75 : 76;
  }
  if (variant == VAR_F8_SYNC) {
    // wide N: 128-row tiles from M = 33, the split 256-row tiles from M = 193
    // (tuner: M = 64 46.7 vs 53.6 us, M = 128 24-30 %, M = 1024 10.5 %)
    if ((wide && M > 32) || (long_k && M > 128)) {
      if (M <= 128 || (!wide && M > 512)) return 54;  // 14B, M = 768: 160.5 vs 192.8 us
      return M <= 768 && tile_rounds(M, N, K, 128, 128, false, cus) <
                             tile_rounds(M, N, K, 256, 128, true, cus)
                 ? 54 : 53;
    }
    // mid-width N around M = 768: three 256-row bands fill one round where
    // six 128-row bands need two (tuner, 1.5B: 36.3 vs 41.3 us; 3B 3 %)
    if (mid && K < 4096 && M > 640 && M <= 1024) return 53;
    return M <= 192 ? 55 : (M <= 3072 ? 54 : 53);
  }
  if (variant == VAR_F8) {
    // FP8: split-K weight streaming up to M = 64, then 64 x 128 tiles, 128-row
    // tiles around M = 256, and the eight-wave 256 x 256 tiles (split tail)
    // (measured: M = 16 and 32 at K = 3584, N = 18944; M = 64 there and at
    // K = 896, N = 4864; M = 128 at the 0.5B shape)
    // (narrow N at M <= 16: fewer than two one-wave workgroups per CU, the
    // split-K configuration wins: 7B decode share 12.2 vs 15.7 us)
    if (M <= 16) return (2 * N + 31) / 32 >= 2 * cus ? 52 : 51;
    // 17-32 rows on narrower matrices: the 64 x 128 tile (1.5B: 11.6 vs 15.6 us)
    if (M <= 32) return wide ? 51 : 46;
    // wide N from M = 33: 128-row tiles, or the split 256-row tiles where
    // they take fewer weighted rounds (M = 192: 52.9 vs 71.9 us; M = 320:
    // 128-row 71.7 vs 91.8 us)
    if ((wide && M > 32) || (long_k && M > 128 && M <= 512)) {
      if (M <= 128) return 45;
      return M <= 768 && tile_rounds(M, N, K, 128, 128, false, cus) <
                             tile_rounds(M, N, K, 256, 128, true, cus)
                 ? 45 : 43;
    }
    return M <= 192 ? 46 : ((M <= 384 || few_big) ? 45 : 43);
  }
  if (M <= 64 && M > 16 && wide) {
    // 17-64 rows on wide matrices: the LDS-tiled kernels beat split-K
    // streaming (tuner, 7B: interleave 128 x 256 at M = 32 54.8 vs 72.5 us,
    // 256 x 192 at M = 64 60.3 vs 84.7 us; sync 128 x 128 73.2 vs 79.1 us and
    // 82.3 vs 93.5 us; GEMM 128 x 128 73.9 vs 76.4 us and 85.4 vs 89.7 us)
    if (variant == VAR_GEMM) return 16;
    if (variant == VAR_SYNC) return 8;
    return M <= 32 ? 1 : 35;
  }
  if (M <= 64 && M > 16 && variant != VAR_SYNC) {
    // 17-64 rows on narrower matrices: the small LDS-tiled tiles beat split-K
    // streaming (tuner, 0.5B and 1.5B K and N: interleave 64 x 128 with 8
    // stages at M = 32 7-8 %, 64 x 128 at M = 64 16-24 %; GEMM 64 x 64 with 8
    // stages 28-32 %)
    if (variant == VAR_GEMM) return 30;
    return M <= 32 ? 27 : 3;
  }
  if (M <= 64 && variant == VAR_GEMM && !wide) return 30;  // 25 % at M = 16
  if (M <= 64) {
    // decode-sized batches: split-K weight streaming, 16-row MFMA blocks
    const int mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    return find_config(variant, 1, mt * 16, variant == VAR_GEMM ? 128 : 64, 0);
  }
  // LDS-tiled, by M (measured at K = 1536, N = 8960 for M = 256 ... 8192 and
  // on the workload shapes): 64-row tiles with deep stage rings around
  // M = 128, 128-row tiles around M = 256, and from M = 512 on the 256-row
  // eight-wave tiles (4x2 waves, short last round split into quarter tiles),
  // which won even where they leave CUs idle (M = 512: 140 tiles on 256 CUs).
  // narrow N (few_big above): the 128-row tiles
  if (variant == VAR_GEMM) {
    // wide N (tuner, 7B and 72B): 128 x 128 to M = 128 (21-39 %), 256 x 128
    // to M = 256 (19 %, 8.7 % at M = 192), 256 x 192 to M = 512 (32.5 % at
    // M = 384, 5 % at M = 512)
    if (wide) return M <= 128 ? 16 : (M <= 256 ? 15 : (M <= 512 ? 22 : 41));
    // mid-width N: 64 x 64 with the shallow ring to M = 96, split-K streaming
    // 64 x 128 to M = 128 (8.5-10 %), 128 x 128 to M = 192 (3B: 49.7 vs
    // 59.5 us at M = 160), and 256 x 128 from M = 385 while those tiles fit
    // in two rounds (1.5B: 72.7 vs 85.1 us at M = 512, 76.5 vs 88.4 us at
    // M = 768; 3B at M = 768 needs three: 144.2 vs 107.8 us for 256 x 256)
    // long K: 256 x 128 to M = 384, 256 x 192 from M = 641 (14B: 170.8 vs
    // 245.2 us at M = 384, 234.3 vs 252.2 us at M = 768)
    if (long_k && M > 256 && M <= 384) return 15;
    if (long_k && M > 640) return 22;
    if (mid && M <= 96) return 17;
    if (mid && M <= 128) return 20;
    if (mid && M <= 192 && (M > 160 || !one_round64)) return 16;
    if (mid && M > 384 && ((M + 255) / 256) * ((N + 127) / 128) <= cus) return 15;
    return M <= 192 ? 30 : (M <= 384 ? 16 : 41);
  }
  if (variant == VAR_SYNC) {
    // wide N (tuner): 128 x 128 to M = 128 (24-44 %), then 128-row or split
    // 256-row tiles by weighted rounds (M = 192: 256-row 126.6 vs 142.6 us;
    // M = 320 and 384: 128-row 150.7 and 163.0 vs 173.6 and 205.9 us)
    if (wide || (long_k && M > 128)) {
      if (M <= 128 || (!wide && M > 512)) return 8;  // 14B, M = 768: 339.9 vs 357.7 us
      return M <= 768 && tile_rounds(M, N, K, 128, 128, false, cus) <
                             tile_rounds(M, N, K, 256, 128, true, cus)
                 ? 8 : 42;
    }
    // mid-width N: 128 x 64 to M = 128 (3B: 43.0 vs 53.3 us), then 64 x 64
    // while those fit one round, else 128 x 128 (3B, M = 160: 44.4 vs 61.3 us)
    if (mid && M <= 192) return M <= 128 ? 9 : ((M <= 160 && one_round64) ? 10 : 8);
    // narrower matrices to M = 96: split-K streaming, 32-row blocks (0.5B:
    // 11.3 vs 14.0 us at M = 96)
    if (!wide && !mid && M <= 96) return 12;
    // narrower matrices with a long K loop, M = 97 ... 128: split-K streaming,
    // 64-row blocks (72B share under 4-way tensor parallelism: 97.1 vs 109.7 us)
    if (half_long_k && M <= 128) return 13;
    // narrower still (72B 8-way share, N = 3696): 32-row blocks (82.4 vs 116.2 us)
    if (!wide && !mid && K >= 4096 && M <= 128) return 12;
    return M <= 192 ? 29 : ((M <= 384 || few_big) ? 8 : 42);
  }
  if (wide && M <= 256) return M <= 192 ? (K >= 4096 ? 31 : 35) : 21;
  // long K on mid-width N: 256 x 128 (split only from M = 385), 256 x 192 from
  // M = 641 (14B: M = 384 114.3 vs 187.2 us, M = 768 225.7 vs 245.5 us)
  if (long_k && M > 256) return M <= 384 ? 31 : (M <= 640 ? 40 : 21);
  if (wide)  // 128 x 256 or the split 256-row tiles by weighted rounds
    return M <= 768 && tile_rounds(M, N, K, 128, 128, false, cus) <
                           tile_rounds(M, N, K, 256, 128, true, cus)
               ? 1 : 40;
  // mid-width N: 128 x 64 to M = 128, 128 x 128 to M = 192 (1.5B M = 96
  // 21.7 vs 27.3 us; 3B M = 160 33.6 vs 41.7 us, M = 192 37.1 vs 45.1 us)
  if (mid && M <= 192) return M <= 128 ? 2 : 1;
  // narrower matrices, M = 65 ... 96: 64 x 64 with the deep stage ring (7B
  // share under 8-way tensor parallelism, M = 96: 25.8 vs 30.7 us)
  if (!wide && !mid && M <= 96) return 27;
  // narrower matrices with a long K loop, M = 257 ... 768: 256 x 192 tiles
  // (72B share under 4-way tensor parallelism: M = 384 134.3 vs 142.3 us,
  // M = 768 170.3 vs 185.5 us)
  if (half_long_k && M > 256 && M <= 768) return 21;
  return M <= 192 ? 3 : ((M <= 384 || few_big) ? 1 : 40);
}

int recommend_layout(long long M, long long N, long long K, int cu_count) {
  (void)K;
  // The page prefers the sync kernel above M = 2048.  On MI355X the interleave
  // kernel was faster at every measured M (0.5B-72B shapes, M = 16..8192): it
  // loads A once and keeps every accumulator busy in every K step, while the
  // sync kernel alternates between half of its registers (Gate, then Up).
  // Up to M = 64 the same Kernel-2 order on fragment-ordered weights streams
  // them fastest (1.16-1.6x the interleaved layout at M = 16 ... 64), except
  // on wide matrices above M = 16, where the LDS-tiled kernel wins (7B: 54.8
  // vs 59.7 us at M = 32, 60.3 vs 74.5 us at M = 64).
  const long long cus = cu_count > 0 ? cu_count : 256;
  const bool wide = (2 * N + 255) / 256 * 2 >= cus;
  if (M <= 16 || (M <= 64 && !wide)) return 2;
  return 1;
}

}  // namespace swiglu
