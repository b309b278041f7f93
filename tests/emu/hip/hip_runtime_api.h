// Host stand-in for the HIP runtime API, used only by the CPU bounds
// emulation of the kernels (tests/emu): enough for swiglu_internal.h and the
// launch functions in swiglu_kernels.hip.
#pragma once
#include <stddef.h>
#include <stdint.h>

struct dim3 {
  unsigned x, y, z;
  constexpr dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1 };
typedef struct emu_stream* hipStream_t;
inline hipError_t hipGetLastError() { return hipSuccess; }
