// swiglu_device.hpp -- gfx950 device building blocks for the fused SwiGLU GEMMs.
//
// MFMA operand conventions used throughout (CDNA3/CDNA4 matrix-core layout,
// 64-lane waves; the k placement only has to agree between the two sources):
//   v_mfma_f32_32x32x16_bf16  A: lane l holds row l%32, k = 8*(l/32) + [0,8)
//                             B: lane l holds col l%32, k = 8*(l/32) + [0,8)
//                             D: lane l, reg r -> col l%32,
//                                row 8*(r/4) + 4*(l/32) + r%4
//   v_mfma_f32_16x16x32_bf16  A: lane l holds row l%16, k = 8*(l/16) + [0,8)
//                             B: lane l holds col l%16, k = 8*(l/16) + [0,8)
//                             D: lane l, reg r -> col l%16, row 4*(l/16) + r
// Both sources want 8 consecutive k per lane.  A [M,K] is k-contiguous in HBM;
// the weights [K,N] are n-contiguous, so the LDS-tiled kernels read weight
// fragments with the transposing LDS read, the strided streaming kernel
// transposes 8x8 blocks of bf16 in registers (v_perm_b32), and the
// fragment-ordered layouts store the weights k-contiguous in the first place.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swiglu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 load8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
// Streaming loads of data that is read exactly once (weights at decode-sized
// batches): the nontemporal hint keeps them from displacing reusable lines.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 load8_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// ---- direct HBM -> LDS loads ------------------------------------------------
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Byte offset that lies past every buffer resource used here (tensors are
// limited to < 2^31 bytes): a load at this offset returns zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Raw buffer resource over [p, p + bytes): stride 0, bounds-checked by byte
// offset (loads past num_records return 0), gfx9 default data format word.
__device__ __forceinline__ i32x4 make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)((a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  r[3] = 0x00020000;
  return r;
}

// LDS address (byte offset in the workgroup's LDS) of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 16-byte-per-lane DMA from global memory into LDS: lane i's 16 bytes land
// at lds_wave_base + 16 i (lds_wave_base is wave-uniform).  Issued as inline
// assembly so the compiler does not add a conservative vmcnt(0) in front of
// every LDS read; completion is tracked with wait_vmcnt<>() by the caller.
__device__ __forceinline__ void lds_dma16(uint32_t lds_wave_base, uint32_t voffset, i32x4 rsrc) {
  // both operands are wave-uniform by construction; readfirstlane makes that
  // visible to the compiler where its divergence analysis cannot prove it
  lds_wave_base = __builtin_amdgcn_readfirstlane(lds_wave_base);
#pragma unroll
  for (int i = 0; i < 4; ++i) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
  // the compiler itself places the LDS base in M0 (the "{m0}" operand)
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds_wave_base)
               : "memory");
}

// Cross-workgroup handoff of fp32 partial sums (the split-K decode kernel).
// The partials are written and read with agent-scope atomic stores and loads
// (device-coherent accesses, which do not stay in one XCD's L2), so no
// cache-wide writeback or invalidate is needed: after its partial stores
// have completed (s_waitcnt vmcnt(0)) a workgroup increments the counter, and
// the last one to arrive reads every partial with agent-scope loads.
__device__ __forceinline__ void store_agent(f32x4* p, f32x4 v) {
  float* f = reinterpret_cast<float*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) __hip_atomic_store(f + i, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 load_agent(const f32x4* p) {
  const float* f = reinterpret_cast<const float*>(p);
  f32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __hip_atomic_load(f + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}
__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Transposing LDS read (gfx950): within each group of 16 lanes, source lane
// s supplies 4 consecutive 16-bit elements at its address, and lane 4a+b
// receives element b of source lanes a, 4+a, 8+a, 12+a.  With source lane s
// pointing at row (s/4) and columns 4*(s%4)..+3 of a row-major [k][n] tile,
// lane i of the group receives column i at rows 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// SiLU(x) = x * sigmoid(x) = x / (1 + e^-x) in fp32 on the hardware exp and
// reciprocal (each within about an ulp).  x << 0: e^-x -> +inf, rcp -> 0,
// result -0; x >> 0: result x.  No NaN for finite x.
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)bf16_bits(lo) | ((uint32_t)bf16_bits(hi) << 16);
}
__device__ __forceinline__ float bf16_to_float(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// Transpose an 8 (k) x 8 (n) block of bf16.  row[i] holds k-row i as four
// dwords, dword j = (n = 2j low half, n = 2j+1 high half).  col[c] receives
// column n = c as four dwords, dword p = (k = 2p low, k = 2p+1 high), i.e. the
// 8 consecutive k of one column that an MFMA source lane wants.
__device__ __forceinline__ void transpose8x8(const u32x4 row[8], u32x4 col[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = row[2 * p][j];      // k = 2p
      const uint32_t hi = row[2 * p + 1][j];  // k = 2p+1
      // even column 2j: low halves of both; odd column 2j+1: high halves.
      col[2 * j][p] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      col[2 * j + 1][p] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
    }
  }
}

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// v_mfma_scale_f32_32x32x64_f8f6f4 with both sources in E4M3 (format 0) and
// unit block scales (E8M0 exponent 127 = 2^0): D = A B + C over 64 k.  Each
// source lane holds 32 bytes (one row or column, 32 of the 64 k) as two
// 16-byte halves; the output layout is that of v_mfma_f32_32x32x16_bf16.
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma32_f8(const u32x4 (&a)[2], const u32x4 (&b)[2],
                                            const f32x16& c) {
  const i32x8 x = __builtin_bit_cast(i32x8, __builtin_shufflevector(a[0], a[1], 0, 1, 2, 3, 4, 5, 6, 7));
  const i32x8 y = __builtin_bit_cast(i32x8, __builtin_shufflevector(b[0], b[1], 0, 1, 2, 3, 4, 5, 6, 7));
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 127, 0, 127);
}

// The same with E8M0 block scales (2^(e - 127)) taken from the low byte of a
// per-lane value: sw scales the first source, sa the second.  Lane l's scale
// covers the k block of 32 that lanes l % 32 and l % 32 + 32 hold in bytes
// 16 (l / 32) .. 16 (l / 32) + 15 of their fragments (block 0: bytes 0-15 of
// both lane halves, block 1: bytes 16-31), for row or column l % 32.
// SEL0 / SEL1 pick the byte of sa_src0 / sb_src1 that holds the scale.
template <int SEL0, int SEL1>
__device__ __forceinline__ f32x16 mfma32_f8_scaled(const u32x4 (&a)[2], const u32x4 (&b)[2],
                                                   const f32x16& c, uint32_t sa_src0,
                                                   uint32_t sb_src1) {
  const i32x8 x = __builtin_bit_cast(i32x8, __builtin_shufflevector(a[0], a[1], 0, 1, 2, 3, 4, 5, 6, 7));
  const i32x8 y = __builtin_bit_cast(i32x8, __builtin_shufflevector(b[0], b[1], 0, 1, 2, 3, 4, 5, 6, 7));
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, SEL0, (int)sa_src0, SEL1,
                                                          (int)sb_src1);
}

// v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 sources and unit block scales:
// each source lane holds 32 bytes (one row or column, 32 of the 128 k); the
// output layout is that of v_mfma_f32_16x16x32_bf16.
__device__ __forceinline__ f32x4 mfma16_f8(const u32x4 (&a)[2], const u32x4 (&b)[2],
                                           const f32x4& c) {
  const i32x8 x = __builtin_bit_cast(i32x8, __builtin_shufflevector(a[0], a[1], 0, 1, 2, 3, 4, 5, 6, 7));
  const i32x8 y = __builtin_bit_cast(i32x8, __builtin_shufflevector(b[0], b[1], 0, 1, 2, 3, 4, 5, 6, 7));
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 0, 127, 0, 127);
}

// fp32 -> OCP E4M3 code, round to nearest even, saturating: |v| >= 448 (and
// infinities) -> +-448, NaN -> S.1111.111; the sign of zero is kept.  Below
// 2^-6 the codes count multiples of 2^-9; above, the 3-bit mantissa is the
// rounded number of eighths of 2^e, and a carry to 16 eighths moves into the
// next binade by itself (code arithmetic).  Scaling by powers of two is exact.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__builtin_bit_cast(uint32_t, v) >> 24) & 0x80u;
  const float a = __builtin_fabsf(v);
  uint32_t code;
  if (!(a == a)) {
    code = 0x7Fu;
  } else if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const int e = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xffu) - 127;
    const float q = __builtin_rintf(__builtin_ldexpf(a, 3 - e));  // 8 .. 16
    code = (uint32_t)((e + 7) << 3) + (uint32_t)q - 8u;
  }
  return sign | code;
}

// Workgroup id -> tile id so that each of the 8 XCDs (which receive workgroups
// round-robin in launch order) works on one contiguous range of tile ids, and
// the tiles that run together on an XCD share operand panels in its L2.
__device__ __forceinline__ int xcd_remap(int b, int nwg) {
  const int q = nwg / 8, r = nwg % 8;
  const int x = b % 8, i = b / 8;
  return x * q + (x < r ? x : r) + i;
}

}  // namespace swiglu
