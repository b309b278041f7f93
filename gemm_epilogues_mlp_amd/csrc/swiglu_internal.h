// swiglu_internal.h -- declarations shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace swiglu {

// VAR_F8 / VAR_F8_SYNC: interleave / sync order on FP8 (E4M3) inputs with
// k-contiguous paired weights
// VAR_MX: interleave order on MXFP8 inputs (E4M3 + E8M0 scale per 32 along K)
// VAR_PACKED: interleave order on W_fused stored in MFMA fragment order
// VAR_F8_PACKED: interleave order on FP8 inputs with fragment-ordered W8
// VAR_MX_PACKED: interleave order on MXFP8 inputs, W8 in the 32x32x64 fragment order
// VAR_MX_SYNC: sync order on MXFP8 inputs (the same W8 and scales as VAR_MX)
// VAR_PACKED_SPLITK: VAR_PACKED with K also split over workgroups (M <= 16;
// needs a workspace, swiglu_forward_packed_splitk only)
enum Variant {
  VAR_AUTO = 0, VAR_SYNC = 1, VAR_INTERLEAVE = 2, VAR_GEMM = 3, VAR_F8 = 4, VAR_F8_SYNC = 5,
  VAR_MX = 6, VAR_PACKED = 7, VAR_F8_PACKED = 8, VAR_MX_PACKED = 9, VAR_MX_SYNC = 10,
  VAR_PACKED_SPLITK = 11
};

// Fragment-ordered W_fused: slabs of 128 columns times steps of 32 k, 4096
// values per (slab, step) block.
inline long long packed_slabs(long long N) { return (2 * N + 127) / 128; }
inline long long packed_steps(long long K) { return (K + 31) / 32; }
inline long long packed_elems(long long N, long long K) {
  return packed_slabs(N) * packed_steps(K) * 4096;
}
// Fragment-ordered W8 (FP8): blocks of 16 rows of the 2N x K pairing times
// steps of 128 k, 2048 bytes per block.
inline long long f8_packed_bytes(long long N, long long K) {
  return ((2 * N + 15) / 16) * ((K + 127) / 128) * 2048;
}
// Fragment-ordered W8 (MXFP8, K % 64 == 0): blocks of 32 rows times steps of
// 64 k, 2048 bytes per block.
inline long long mx_packed_bytes(long long N, long long K) {
  return ((2 * N + 31) / 32) * (K / 64) * 2048;
}

// Workspace of the split-K streaming kernel for `slabs` slabs of W_fused and
// S pieces of K: a uint32 counter per (slab, part) -- slabs * 4 reserved,
// rounded to 256 bytes -- then the fp32 partials, 8 KB per slab and piece.
inline long long splitk_counter_bytes(long long slabs) { return (slabs * 16 + 255) / 256 * 256; }
inline long long splitk_workspace_bytes(long long slabs, long long S) {
  return splitk_counter_bytes(slabs) + slabs * S * 8192;
}

struct LaunchArgs {
  const uint16_t* A;
  const uint16_t* W1;  // W1, W_fused, or the single GEMM weight
  const uint16_t* W2;  // W2 (sync) or unused
  uint16_t* Y;         // Y, or G / U for the unfused GEMMs
  int M, N, K;         // N = output columns (Y columns, or G columns)
  int ldw, ldy;        // row strides (elements) of the weights and of Y
  int group_m;         // tile rows per GROUP_M band (<= 0: default)
  int cu_count;        // compute units of the device (workgroups per round)
  float scale_g, scale_u;  // FP8: s_a * s_w1 and s_a * s_w2 (unused otherwise)
  const uint8_t* SA;       // MXFP8: E8M0 scales of A [M, ks] and of W8 [2N, ks]
  const uint8_t* SW;
  int ks;                  // MXFP8: scale row stride (bytes, a multiple of 16)
  hipStream_t stream;
  void* ws = nullptr;      // split-K streaming: workspace (splitk_workspace_bytes)
  int ksplit = 1;          // split-K streaming: workgroups per (slab, part) along K
};

typedef hipError_t (*LaunchFn)(const LaunchArgs&);

struct KernelConfig {
  int variant;  // Variant
  int family;   // 0 tiled, 1 streaming, 2 persistent tiled, 3 streaming split over workgroups
  int bm, bn, bk, waves, split_k, lds_bytes;
  LaunchFn launch;
  int tail_split;  // 0, or 4: big tiles of a partial last round run as quarter tiles
};

int config_count();
const KernelConfig* config_at(int id);

hipError_t launch_gate(const uint16_t* G, const uint16_t* U, uint16_t* Y, size_t n,
                       hipStream_t stream, int cu_count);
hipError_t launch_pack(const uint16_t* W1, const uint16_t* W2, uint16_t* WF, size_t n,
                       hipStream_t stream, int cu_count);
// FP8: bf16 -> E4M3 of x * inv_scale (n a multiple of 16); W1, W2 [K, N] E4M3 ->
// W8 [2N, K] (K a multiple of 16)
hipError_t launch_quantize_f8(const uint16_t* X, uint8_t* Q, size_t n, float inv_scale,
                              hipStream_t stream, int cu_count);
hipError_t launch_pack_f8(const uint8_t* W1, const uint8_t* W2, uint8_t* W8, int N, int K,
                          hipStream_t stream, int cu_count);
// MXFP8: bf16 rows [rows, K] -> E4M3 [rows, K] + E8M0 [rows, ks]; bf16 W1, W2
// [K, N] -> Wt [2N, K] (k-major pairing)
hipError_t launch_quantize_mx(const uint16_t* X, uint8_t* Q, uint8_t* S, int rows, int K, int ks,
                              hipStream_t stream, int cu_count);
// E4M3 W8 [R = 2N, K] -> MX fragment-ordered W8 (mx_packed_bytes(N, K) bytes)
hipError_t launch_pack_mx_frag(const uint8_t* W8, uint8_t* P, int R, int K, hipStream_t stream,
                              int cu_count);
// E4M3 W8 [R = 2N, K] -> fragment-ordered W8 (f8_packed_bytes(N, K) bytes)
hipError_t launch_pack_f8_frag(const uint8_t* W8, uint8_t* P, int R, int K, hipStream_t stream,
                              int cu_count);
// bf16 W1, W2 [K, N] -> fragment-ordered W_fused (packed_elems(N, K) values)
hipError_t launch_pack_frag(const uint16_t* W1, const uint16_t* W2, uint16_t* P, int N, int K,
                           hipStream_t stream, int cu_count);
hipError_t launch_pack_kmajor(const uint16_t* W1, const uint16_t* W2, uint16_t* Wt, int N, int K,
                              hipStream_t stream, int cu_count);

// Per-shape choice (tile table + fallback rule).  variant is SYNC, INTERLEAVE
// or GEMM; returns a config id of that variant.
int select_config(int variant, long long M, long long N, long long K, int cu_count);
// Layout the table recommends for a shape: 0 separate, 1 interleaved, 2 packed.
int recommend_layout(long long M, long long N, long long K, int cu_count);

}  // namespace swiglu
