// Host stand-in for swiglu_device.hpp: the same names and signatures, with
// every LDS and global access bounds-checked instead of executed on a GPU.
// Used only by the CPU bounds emulation (tests/emu); numerical results are
// not produced (the MFMAs return their accumulator unchanged).
//
// LDS: the emulation rewrites each kernel's shared array into a call to
// emu_lds(bytes), which returns one heap buffer of exactly that size; LDS
// "addresses" are byte offsets into it.  Global memory: the driver registers
// every buffer it passes in; a DMA or load from outside a registered buffer
// is reported (on the GPU it would be a memory fault).
#pragma once

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "hip/hip_runtime_api.h"

// ---- emulation state (defined in emu_driver.cpp) ------------------------------
extern dim3 threadIdx, blockIdx, gridDim, blockDim;
uint8_t* emu_lds(size_t bytes);
void emu_barrier();
void emu_check_global(const void* p, size_t n, const char* what);
void emu_check_lds(uint32_t off, size_t n, const char* what);
uint8_t* emu_lds_base();
// LDS ordering check (emu_race.cpp)
void emu_race_block_begin();
void emu_race_thread(unsigned t);
long emu_race_block_end();
void emu_race_barrier();
void emu_race_wait(int n);
void emu_race_vmop();
void emu_race_dma(uint32_t dst, uint32_t n);
void emu_race_read(const void* p, uint32_t n);
extern long g_emu_race_errors;
extern int g_emu_plant;  // a planted mistake to switch on (build.py), 0: none
// byte copies outside the instrumented translation unit (so that the data
// movement of a DMA or of a checked load is not logged as a plain access)
void emu_copy(void* d, const void* s, size_t n);
void emu_use(const void* p, size_t n);
void emu_zero(void* d, size_t n);

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
inline void __syncthreads() { emu_barrier(); }
// device-side integer min/max as HIP provides them
inline int min(int a, int b) { return a < b ? a : b; }
inline int max(int a, int b) { return a > b ? a : b; }
#define __builtin_amdgcn_readfirstlane(x) (x)
#define __builtin_amdgcn_sched_barrier(x) ((void)0)
inline uint32_t emu_perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  const uint64_t v = ((uint64_t)s0 << 32) | s1;
  uint32_t r = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = (sel >> (8 * i)) & 0xff;
    const uint32_t byte = b < 8 ? (uint32_t)((v >> (8 * b)) & 0xff) : 0u;
    r |= byte << (8 * i);
  }
  return r;
}
#define __builtin_amdgcn_perm(a, b, s) emu_perm((a), (b), (s))

// emulate only the last g_emu_last_blocks workgroups of each launch (0: all);
// the last workgroups of a launch touch the largest offsets.  The LDS
// ordering check runs on the last g_emu_race_blocks of them (0: all).
extern long g_emu_last_blocks;
extern long g_emu_race_blocks;
void emu_race_enable(bool on);
bool emu_race_enabled();
template <class K, class... Args>
void emu_launch(K kernel, dim3 grid, dim3 block, Args... args) {
  gridDim = grid;
  blockDim = block;
  const long total = (long)grid.x * grid.y;
  const long first = g_emu_last_blocks > 0 && g_emu_last_blocks < total ? total - g_emu_last_blocks : 0;
  const long race_first = g_emu_race_blocks > 0 && g_emu_race_blocks < total ? total - g_emu_race_blocks : 0;
  const bool race_on = emu_race_enabled();
  for (unsigned by = 0; by < grid.y; ++by)
    for (unsigned bx = 0; bx < grid.x; ++bx) {
      if ((long)by * grid.x + bx < first) continue;
      blockIdx = dim3(bx, by, 0);
      emu_race_enable(race_on && (long)by * grid.x + bx >= race_first);
      emu_race_block_begin();
      for (unsigned t = 0; t < block.x; ++t) {
        threadIdx = dim3(t, 0, 0);
        emu_race_thread(t);
        kernel(args...);
      }
      g_emu_race_errors += emu_race_block_end();
      emu_race_enable(race_on);
    }
}
#define hipLaunchKernelGGL(K, G, B, SHM, STREAM, ...) emu_launch(K, dim3(G), dim3(B), __VA_ARGS__)

namespace swiglu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

inline u32x4 load16(const void* p) {
  emu_check_global(p, 16, "load16");
  emu_race_vmop();
  u32x4 r;
  emu_copy(&r, p, 16);
  return r;
}
inline u32x2 load8(const void* p) {
  emu_check_global(p, 8, "load8");
  emu_race_vmop();
  u32x2 r;
  emu_copy(&r, p, 8);
  return r;
}
inline u32x4 load16_stream(const void* p) { return load16(p); }
inline u32x2 load8_stream(const void* p) { return load8(p); }

constexpr uint32_t kOutOfRange = 0x80000000u;

// the resource keeps the full host pointer (words 0-1) and the byte bound (2)
inline i32x4 make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  i32x4 r;
  r[0] = (int32_t)(uint32_t)a;
  r[1] = (int32_t)(uint32_t)(a >> 32);
  r[2] = (int32_t)bytes;
  r[3] = 0x00020000;
  return r;
}
inline uint32_t lds_addr(const void* p) {
  const uint8_t* b = emu_lds_base();
  const ptrdiff_t d = (const uint8_t*)p - b;
  emu_check_lds((uint32_t)d, 0, "lds_addr");
  return (uint32_t)d;
}
// lane = threadIdx.x % 64 moves 16 bytes from base + voffset (zeros if
// voffset >= the resource bound) to LDS offset lds_wave_base + 16 lane
inline void lds_dma16(uint32_t lds_wave_base, uint32_t voffset, i32x4 rsrc) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t dst = lds_wave_base + 16u * lane;
  emu_check_lds(dst, 16, "lds_dma16 destination");
  emu_race_dma(dst, 16);
  uint8_t* d = emu_lds_base() + dst;
  const uint32_t bound = (uint32_t)rsrc[2];
  if (voffset >= bound) {
    emu_zero(d, 16);
    return;
  }
  if (voffset + 16u > bound) emu_check_global(nullptr, 0, "lds_dma16 read straddles the resource bound");
  const uint8_t* base =
      (const uint8_t*)(uintptr_t)(((uint64_t)(uint32_t)rsrc[1] << 32) | (uint32_t)rsrc[0]);
  emu_check_global(base + voffset, 16, "lds_dma16 source");
  emu_copy(d, base + voffset, 16);
}
// cross-workgroup handoff: the workgroups run one after another here, so the
// coherent accesses are plain copies (their addresses checked) and the
// counter a plain add
inline void store_agent(f32x4* p, f32x4 v) {
  emu_check_global(p, 16, "store_agent");
  emu_copy(p, &v, 16);
}
inline f32x4 load_agent(const f32x4* p) {
  emu_check_global(p, 16, "load_agent");
  emu_race_vmop();
  f32x4 v;
  emu_copy(&v, p, 16);
  return v;
}
inline uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  emu_check_global(p, 4, "atomic_add_agent");
  const uint32_t old = *p;
  *p = old + v;
  return old;
}
template <int N>
inline void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  emu_race_wait(N);
}
inline u32x2 lds_read_tr16(const void* p) {
  const uint8_t* b = emu_lds_base();
  emu_check_lds((uint32_t)((const uint8_t*)p - b), 8, "lds_read_tr16");
  emu_race_read(p, 8);
  u32x2 r;
  emu_copy(&r, p, 8);
  return r;
}
inline float silu(float x) { return x / (1.0f + expf(-x)); }
inline uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x)); }
inline uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)bf16_bits(lo) | ((uint32_t)bf16_bits(hi) << 16);
}
inline float bf16_to_float(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }
inline void transpose8x8(const u32x4 row[8], u32x4 col[8]) {
  for (int j = 0; j < 4; ++j)
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = row[2 * p][j], hi = row[2 * p + 1][j];
      col[2 * j][p] = emu_perm(hi, lo, 0x05040100u);
      col[2 * j + 1][p] = emu_perm(hi, lo, 0x07060302u);
    }
}
// The matrix products are not computed (values are the GPU tests' job), but
// their operands are handed to emu_use, a function of another translation
// unit: otherwise the compiler drops every LDS read whose only use is an MFMA
// operand, and the LDS ordering check never sees those reads.
inline f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  emu_use(&a, 16), emu_use(&b, 16);
  return c;
}
inline f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  emu_use(&a, 16), emu_use(&b, 16);
  return c;
}
inline f32x16 mfma32_f8(const u32x4 (&a)[2], const u32x4 (&b)[2], const f32x16& c) {
  emu_use(a, 32), emu_use(b, 32);
  return c;
}
inline f32x4 mfma16_f8(const u32x4 (&a)[2], const u32x4 (&b)[2], const f32x4& c) {
  emu_use(a, 32), emu_use(b, 32);
  return c;
}
template <int SEL0, int SEL1>
inline f32x16 mfma32_f8_scaled(const u32x4 (&a)[2], const u32x4 (&b)[2], const f32x16& c,
                               uint32_t sa, uint32_t sb) {
  static_assert(SEL0 >= 0 && SEL0 < 4 && SEL1 >= 0 && SEL1 < 4, "byte select");
  emu_use(a, 32), emu_use(b, 32), emu_use(&sa, 4), emu_use(&sb, 4);
  return c;
}
inline uint32_t e4m3_code(float v) {
  uint32_t bits;
  memcpy(&bits, &v, 4);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(v);
  if (!(a == a)) return sign | 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);
  uint32_t ab;
  memcpy(&ab, &a, 4);
  const int e = (int)((ab >> 23) & 0xffu) - 127;
  return sign | ((uint32_t)((e + 7) << 3) + (uint32_t)rintf(ldexpf(a, 3 - e)) - 8u);
}
inline int xcd_remap(int b, int nwg) {
  const int q = nwg / 8, r = nwg % 8;
  const int x = b % 8, i = b / 8;
  return x * q + (x < r ? x : r) + i;
}

}  // namespace swiglu
