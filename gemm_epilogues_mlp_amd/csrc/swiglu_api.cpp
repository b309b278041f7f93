// swiglu_api.cpp -- the extern "C" boundary: argument checks, handle, dispatch.
// Every check runs before anything is enqueued; see include/swiglu.h for the
// contract of each entry point.
#include "swiglu.h"

#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <algorithm>
#include <vector>

#include "swiglu_internal.h"

struct swiglu_tuned_entry {
  int variant;
  long long M, N, K;
  int config_id;
};

struct swiglu_ctx {
  int device;
  int cu_count;
  char arch[64];
  int log;  // SWIGLU_LOG=1: print the configuration chosen for each call
  std::vector<swiglu_tuned_entry> tuned;  // exact-shape overrides, read at creation
  void* scratch;  // this device's copy of the fixed scratch array (device address)
};

// ---- fixed device scratch for callers that cannot allocate -------------------
// swiglu_forward_unfused_static keeps the unfused baseline's bf16 Gate and Up
// tensors here instead of in a caller workspace.  One copy per device, held
// until the process ends; every call on a device shares it.  In host code the
// array's name is only a stand-in: its device address on each device comes
// from hipGetSymbolAddress (resolved once per device in swiglu_create, with
// that device current) and only that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[SWIGLU_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of this device's `scratch` (resolving it on first use);
// nullptr if it cannot be resolved.
void* scratch_address(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[device]) return g_scratch_addr[device];
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return nullptr;
  if (prev != device && hipSetDevice(device) != hipSuccess) return nullptr;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (prev != device) (void)hipSetDevice(prev);
  if (e != hipSuccess || !ptr) return nullptr;
  g_scratch_addr[device] = ptr;
  return ptr;
}
}  // namespace

namespace {

using namespace swiglu;

constexpr long long kMaxDim = 0x7fffffffLL;
constexpr long long kMaxBytes = 1LL << 31;  // each tensor must be smaller

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// [p, p + bytes) and [q, q + qbytes) overlap (empty ranges never do)
bool overlaps(const void* p, long long bytes, const void* q, long long qbytes) {
  if (!p || !q || bytes <= 0 || qbytes <= 0) return false;
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + (uintptr_t)qbytes && b < a + (uintptr_t)bytes;
}

// The configuration for a shape: an exact tuned entry of the handle if there
// is one, else the built-in table and its fallback rule.
int choose(const swiglu_ctx* h, int variant, long long M, long long N, long long K) {
  for (const swiglu_tuned_entry& e : h->tuned)
    if (e.variant == variant && e.M == M && e.N == N && e.K == K) return e.config_id;
  return select_config(variant, M, N, K, h->cu_count);
}

// ---- tuned-configuration files ---------------------------------------------
// Text, one entry per line after a header line
//   swiglu-tuned <signature, 16 hex digits> <arch>
//   <variant> <M> <N> <K> <config id> [anything else: provenance, ignored]
// '#' starts a comment line; blank lines are skipped.
constexpr int kMaxTunedEntries = 4096;

uint64_t config_signature() {
  uint64_t h = 1469598103934665603ull;  // FNV-1a over the configuration list
  auto mix = [&](long long v) {
    for (int i = 0; i < 8; ++i) {
      h ^= (uint64_t)((v >> (8 * i)) & 0xff);
      h *= 1099511628211ull;
    }
  };
  mix(config_count());
  for (int i = 0; i < config_count(); ++i) {
    const KernelConfig* c = config_at(i);
    for (long long v : {(long long)c->variant, (long long)c->family, (long long)c->bm,
                        (long long)c->bn, (long long)c->bk, (long long)c->waves,
                        (long long)c->split_k, (long long)c->lds_bytes, (long long)c->tail_split})
      mix(v);
  }
  return h;
}

swiglu_status_t read_tuned(const char* path, std::vector<swiglu_tuned_entry>* out) {
  if (!path) return SWIGLU_ERR_INVALID_ARG;
  FILE* f = fopen(path, "r");
  if (!f) return SWIGLU_ERR_INVALID_ARG;
  char line[512];
  bool header = false;
  swiglu_status_t st = SWIGLU_OK;
  while (st == SWIGLU_OK && fgets(line, sizeof line, f)) {
    if (!strchr(line, '\n') && !feof(f)) {  // longer than any valid line
      st = SWIGLU_ERR_INVALID_ARG;
      break;
    }
    const char* p = line;
    while (*p == ' ' || *p == '\t') ++p;
    if (*p == '#' || *p == '\n' || *p == '\r' || *p == 0) continue;
    if (!header) {
      unsigned long long sig = 0;
      char arch[64];
      if (sscanf(p, "swiglu-tuned %16llx %63s", &sig, arch) != 2) {
        st = SWIGLU_ERR_INVALID_ARG;
      } else if (sig != config_signature()) {
        st = SWIGLU_ERR_UNSUPPORTED;  // written for another build's configurations
      }
      header = true;
      continue;
    }
    swiglu_tuned_entry e;
    if (sscanf(p, "%d %lld %lld %lld %d", &e.variant, &e.M, &e.N, &e.K, &e.config_id) != 5 ||
        e.M < 0 || e.N < 0 || e.K < 0 || e.M > kMaxDim || e.N > kMaxDim || e.K > kMaxDim) {
      st = SWIGLU_ERR_INVALID_ARG;
      break;
    }
    const KernelConfig* c = config_at(e.config_id);
    if (!c || c->variant != e.variant || (int)out->size() >= kMaxTunedEntries) {
      st = SWIGLU_ERR_INVALID_ARG;
      break;
    }
    out->push_back(e);
  }
  fclose(f);
  if (st == SWIGLU_OK && !header) st = SWIGLU_ERR_INVALID_ARG;
  return st;
}

swiglu_status_t check_device(const swiglu_ctx* h) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return SWIGLU_ERR_DEVICE;
  return cur == h->device ? SWIGLU_OK : SWIGLU_ERR_DEVICE;
}

// Shared argument validation of the forward entry points.  *noop is set when
// there is nothing to compute (M == 0 or N == 0).
swiglu_status_t check_forward(const swiglu_ctx* h, const void* A, const void* W1,
                              const void* W2, const void* Y, int64_t M, int64_t N,
                              int64_t K, int layout, bool* noop) {
  *noop = false;
  if (!h) return SWIGLU_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0) return SWIGLU_ERR_INVALID_ARG;
  if (layout != SWIGLU_LAYOUT_SEPARATE && layout != SWIGLU_LAYOUT_INTERLEAVED &&
      layout != SWIGLU_LAYOUT_PACKED)
    return SWIGLU_ERR_INVALID_ARG;
  if (layout != SWIGLU_LAYOUT_SEPARATE && W2 != nullptr) return SWIGLU_ERR_INVALID_ARG;
  if (M == 0 || N == 0) {
    *noop = true;
    return SWIGLU_OK;
  }
  if (!Y) return SWIGLU_ERR_INVALID_ARG;
  if (K > 0) {
    if (!A || !W1) return SWIGLU_ERR_INVALID_ARG;
    if (layout == SWIGLU_LAYOUT_SEPARATE && !W2) return SWIGLU_ERR_INVALID_ARG;
  }
  if (M > kMaxDim || K > kMaxDim || N > (kMaxDim >> 1)) return SWIGLU_ERR_UNSUPPORTED;
  if (N % 8 != 0 || K % 8 != 0) return SWIGLU_ERR_UNSUPPORTED;
  if (!aligned16(Y) || !aligned16(A) || !aligned16(W1) || !aligned16(W2))
    return SWIGLU_ERR_UNSUPPORTED;
  const long long ybytes = 2LL * M * N;
  const long long abytes = 2LL * M * K;
  const long long wbytes = layout == SWIGLU_LAYOUT_PACKED ? 2LL * packed_elems(N, K)
                           : (layout == SWIGLU_LAYOUT_INTERLEAVED ? 4LL : 2LL) * K * N;
  // the kernels address A and the weights with 32-bit byte offsets, and use
  // offset 2^31 as "past every tensor"
  if (ybytes >= kMaxBytes || abytes >= kMaxBytes || wbytes >= kMaxBytes)
    return SWIGLU_ERR_UNSUPPORTED;
  if (K > 0 && (overlaps(Y, ybytes, A, abytes) || overlaps(Y, ybytes, W1, wbytes) ||
                (layout == SWIGLU_LAYOUT_SEPARATE && overlaps(Y, ybytes, W2, wbytes))))
    return SWIGLU_ERR_INVALID_ARG;
  return check_device(h);
}

// a skinny configuration launches ceil(M / bm) workgroups along grid y
bool config_fits(const KernelConfig* c, long long M) {
  if (c->family == 1) return (M + c->bm - 1) / c->bm <= 65535;
  return true;
}

swiglu_status_t launch(const swiglu_ctx* h, const KernelConfig* cfg, int id,
                       const LaunchArgs& a) {
  if (h->log)
    fprintf(stderr, "[swiglu] M=%d N=%d K=%d -> config %d (variant %d family %d %dx%d)\n", a.M,
            a.N, a.K, id, cfg->variant, cfg->family, cfg->bm, cfg->bn);
  // the launch functions return the status of their own launch (hipLaunchKernel),
  // so an error pending from a caller's earlier HIP call is left alone
  return cfg->launch(a) == hipSuccess ? SWIGLU_OK : SWIGLU_ERR_LAUNCH;
}

swiglu_status_t run(const swiglu_ctx* h, const KernelConfig* cfg, int id, const void* A,
                    const void* W1, const void* W2, void* Y, int64_t M, int64_t N,
                    int64_t K, hipStream_t stream) {
  if (!config_fits(cfg, M)) return SWIGLU_ERR_UNSUPPORTED;
  LaunchArgs a;
  a.A = (const uint16_t*)A;
  a.W1 = (const uint16_t*)W1;
  a.W2 = (const uint16_t*)W2;
  a.Y = (uint16_t*)Y;
  a.M = (int)M, a.N = (int)N, a.K = (int)K;
  a.ldw = cfg->variant == VAR_INTERLEAVE ? (int)(2 * N) : (int)N;
  a.ldy = (int)N;
  a.group_m = 0;
  a.cu_count = h->cu_count;
  a.stream = stream;
  return launch(h, cfg, id, a);
}

// Kernel family of a bf16 layout: SEPARATE -> sync, INTERLEAVED -> interleave,
// PACKED -> interleave on fragment-ordered weights
int layout_family(int layout) {
  if (layout == SWIGLU_LAYOUT_INTERLEAVED) return VAR_INTERLEAVE;
  if (layout == SWIGLU_LAYOUT_PACKED) return VAR_PACKED;
  return VAR_SYNC;
}

// public variants a forward on this layout accepts besides AUTO
bool variant_matches(int layout, int variant) {
  if (layout == SWIGLU_LAYOUT_PACKED)
    return variant == SWIGLU_VARIANT_INTERLEAVE || variant == SWIGLU_VARIANT_PACKED;
  return variant == layout_family(layout);
}

void fill_tile(int id, swiglu_tile_t* t) {
  const KernelConfig* c = config_at(id);
  t->id = id;
  t->variant = c->variant;
  t->family = c->family;
  t->bm = c->bm;
  t->bn = c->bn;
  t->bk = c->bk;
  t->waves = c->waves;
  t->split_k = c->split_k;
  t->lds_bytes = c->lds_bytes;
  t->tail_split = c->tail_split;
}

// FP8 family of a public variant: AUTO and INTERLEAVE -> the interleave
// kernels, SYNC -> the sync kernels; -1 for anything else
int fp8_family(int variant) {
  if (variant == SWIGLU_VARIANT_AUTO || variant == SWIGLU_VARIANT_INTERLEAVE) return VAR_F8;
  if (variant == SWIGLU_VARIANT_SYNC) return VAR_F8_SYNC;
  if (variant == SWIGLU_VARIANT_MXFP8) return VAR_MX;  // queries only
  if (variant == SWIGLU_VARIANT_FP8_PACKED) return VAR_F8_PACKED;
  if (variant == SWIGLU_VARIANT_MXFP8_PACKED) return VAR_MX_PACKED;  // queries only
  if (variant == SWIGLU_VARIANT_MXFP8_SYNC) return VAR_MX_SYNC;      // queries only
  return -1;
}

// The unfused baseline on a Gate/Up buffer `gu` of 4 M N bytes (G then U,
// bf16): two GEMM launches and the separate gate kernel.
swiglu_status_t unfused(const swiglu_ctx* h, const void* A, const void* W1, const void* W2,
                        void* gu, void* Y, int64_t M, int64_t N, int64_t K,
                        int32_t gemm_config_id, hipStream_t stream) {
  bool noop = false;
  swiglu_status_t st =
      check_forward(h, A, W1, W2, Y, M, N, K, SWIGLU_LAYOUT_SEPARATE, &noop);
  if (st != SWIGLU_OK) return st;
  int id = gemm_config_id;
  if (id >= 0) {
    const KernelConfig* c = config_at(id);
    if (!c || c->variant != VAR_GEMM) return SWIGLU_ERR_INVALID_ARG;
  }
  if (noop) return SWIGLU_OK;
  if (!gu) return SWIGLU_ERR_INVALID_ARG;
  if (!aligned16(gu)) return SWIGLU_ERR_UNSUPPORTED;
  const long long wsb = 4LL * M * N;
  const long long wb = 2LL * K * N;
  if (overlaps(gu, wsb, Y, 2LL * M * N) || overlaps(gu, wsb, A, 2LL * M * K) ||
      overlaps(gu, wsb, W1, wb) || overlaps(gu, wsb, W2, wb))
    return SWIGLU_ERR_INVALID_ARG;
  if (id < 0) id = choose(h, VAR_GEMM, M, N, K);
  if (id < 0) return SWIGLU_ERR_UNSUPPORTED;
  uint16_t* G = (uint16_t*)gu;
  uint16_t* U = G + (size_t)M * (size_t)N;
  st = run(h, config_at(id), id, A, W1, nullptr, G, M, N, K, stream);
  if (st != SWIGLU_OK) return st;
  st = run(h, config_at(id), id, A, W2, nullptr, U, M, N, K, stream);
  if (st != SWIGLU_OK) return st;
  if (launch_gate(G, U, (uint16_t*)Y, (size_t)M * (size_t)N, stream, h->cu_count) != hipSuccess)
    return SWIGLU_ERR_LAUNCH;
  return SWIGLU_OK;
}

}  // namespace

extern "C" {

swiglu_status_t swiglu_create(swiglu_handle_t* out, int device) {
  if (!out) return SWIGLU_ERR_INVALID_ARG;
  *out = nullptr;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return SWIGLU_ERR_DEVICE;
  }
  if (device < 0 || device >= count) return SWIGLU_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
    (void)hipGetLastError();
    return SWIGLU_ERR_DEVICE;
  }
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return SWIGLU_ERR_DEVICE;
  swiglu_ctx* h = new (std::nothrow) swiglu_ctx;
  if (!h) return SWIGLU_ERR_ALLOC;
  h->device = device;
  h->cu_count = prop.multiProcessorCount;
  strncpy(h->arch, prop.gcnArchName, sizeof(h->arch) - 1);
  h->arch[sizeof(h->arch) - 1] = 0;
  const char* lg = getenv("SWIGLU_LOG");
  h->log = (lg && lg[0] == '1') ? 1 : 0;
  h->scratch = scratch_address(device);
  if (!h->scratch) {
    delete h;
    return SWIGLU_ERR_DEVICE;
  }
  *out = h;
  return SWIGLU_OK;
}

swiglu_status_t swiglu_destroy(swiglu_handle_t h) {
  delete h;
  return SWIGLU_OK;
}

swiglu_status_t swiglu_forward_ex(swiglu_handle_t h, const void* A, const void* W1,
                                  const void* W2, void* Y, int64_t M, int64_t N, int64_t K,
                                  swiglu_layout_t layout, swiglu_variant_t variant,
                                  int32_t config_id, hipStream_t stream) {
  bool noop = false;
  swiglu_status_t st = check_forward(h, A, W1, W2, Y, M, N, K, (int)layout, &noop);
  if (st != SWIGLU_OK) return st;
  const int want = layout_family((int)layout);
  if (variant != SWIGLU_VARIANT_AUTO && !variant_matches((int)layout, (int)variant))
    return SWIGLU_ERR_INVALID_ARG;
  int id = config_id;
  if (id >= 0) {
    const KernelConfig* c = config_at(id);
    if (!c || c->variant != want) return SWIGLU_ERR_INVALID_ARG;
  }
  if (noop) return SWIGLU_OK;
  if (id < 0) id = choose(h, want, M, N, K);
  if (id < 0) return SWIGLU_ERR_UNSUPPORTED;
  return run(h, config_at(id), id, A, W1, W2, Y, M, N, K, stream);
}

swiglu_status_t swiglu_forward(swiglu_handle_t h, const void* A, const void* W1,
                               const void* W2, void* Y, int64_t M, int64_t N, int64_t K,
                               swiglu_layout_t layout, hipStream_t stream) {
  return swiglu_forward_ex(h, A, W1, W2, Y, M, N, K, layout, SWIGLU_VARIANT_AUTO, -1, stream);
}

int64_t swiglu_unfused_workspace_bytes(int64_t M, int64_t N) {
  if (M < 0 || N < 0) return 0;
  return 4 * M * N;
}

swiglu_status_t swiglu_forward_unfused(swiglu_handle_t h, const void* A, const void* W1,
                                       const void* W2, void* workspace, void* Y, int64_t M,
                                       int64_t N, int64_t K, int32_t gemm_config_id,
                                       hipStream_t stream) {
  return unfused(h, A, W1, W2, workspace, Y, M, N, K, gemm_config_id, stream);
}

swiglu_status_t swiglu_forward_unfused_static(swiglu_handle_t h, const void* A,
                                              const void* W1, const void* W2, void* Y,
                                              int64_t M, int64_t N, int64_t K,
                                              int32_t gemm_config_id, hipStream_t stream) {
  if (!h) return SWIGLU_ERR_INVALID_ARG;
  if (M >= 0 && N >= 0 && N <= (kMaxDim >> 1) && M <= kMaxDim &&
      4LL * M * N > SWIGLU_STATIC_SCRATCH_BYTES) {
    if (h->log)
      fprintf(stderr, "[swiglu] unfused_static: Gate and Up need %lld bytes, the fixed "
              "scratch holds %lld\n", 4LL * M * N, (long long)SWIGLU_STATIC_SCRATCH_BYTES);
    return SWIGLU_ERR_UNSUPPORTED;
  }
  return unfused(h, A, W1, W2, h->scratch, Y, M, N, K, gemm_config_id, stream);
}

swiglu_status_t swiglu_pack_interleaved(swiglu_handle_t h, const void* W1, const void* W2,
                                        void* W_fused, int64_t K, int64_t N,
                                        hipStream_t stream) {
  if (!h || K < 0 || N < 0) return SWIGLU_ERR_INVALID_ARG;
  if (K == 0 || N == 0) return SWIGLU_OK;
  if (!W1 || !W2 || !W_fused) return SWIGLU_ERR_INVALID_ARG;
  if (K > kMaxDim || N > (kMaxDim >> 1)) return SWIGLU_ERR_UNSUPPORTED;
  if (N % 8 != 0) return SWIGLU_ERR_UNSUPPORTED;
  if (!aligned16(W1) || !aligned16(W2) || !aligned16(W_fused)) return SWIGLU_ERR_UNSUPPORTED;
  const long long wb = 2LL * K * N;
  if (overlaps(W_fused, 2 * wb, W1, wb) || overlaps(W_fused, 2 * wb, W2, wb))
    return SWIGLU_ERR_INVALID_ARG;
  swiglu_status_t st = check_device(h);
  if (st != SWIGLU_OK) return st;
  if (launch_pack((const uint16_t*)W1, (const uint16_t*)W2, (uint16_t*)W_fused,
                  (size_t)K * (size_t)N, stream, h->cu_count) != hipSuccess)
    return SWIGLU_ERR_LAUNCH;
  return SWIGLU_OK;
}

int64_t swiglu_fp8_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N > (kMaxDim >> 1) || K > kMaxDim) return 0;
  return f8_packed_bytes(N, K);
}

swiglu_status_t swiglu_pack_fp8_fragments(swiglu_handle_t h, const void* W8, void* P8, int64_t K,
                                          int64_t N, hipStream_t stream) {
  if (!h || K < 0 || N < 0) return SWIGLU_ERR_INVALID_ARG;
  if (K == 0 || N == 0) return SWIGLU_OK;
  if (!W8 || !P8) return SWIGLU_ERR_INVALID_ARG;
  if (K > kMaxDim || N > (kMaxDim >> 1)) return SWIGLU_ERR_UNSUPPORTED;
  if (N % 8 != 0 || K % 16 != 0) return SWIGLU_ERR_UNSUPPORTED;
  if (!aligned16(W8) || !aligned16(P8)) return SWIGLU_ERR_UNSUPPORTED;
  const long long wb = 2LL * K * N, pb = f8_packed_bytes(N, K);
  if (wb >= kMaxBytes || pb >= kMaxBytes) return SWIGLU_ERR_UNSUPPORTED;
  if (overlaps(P8, pb, W8, wb)) return SWIGLU_ERR_INVALID_ARG;
  swiglu_status_t st = check_device(h);
  if (st != SWIGLU_OK) return st;
  if (launch_pack_f8_frag((const uint8_t*)W8, (uint8_t*)P8, (int)(2 * N), (int)K, stream,
                          h->cu_count) != hipSuccess)
    return SWIGLU_ERR_LAUNCH;
  return SWIGLU_OK;
}

int64_t swiglu_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N > (kMaxDim >> 1) || K > kMaxDim) return 0;
  return 2 * packed_elems(N, K);
}

swiglu_status_t swiglu_pack_fragments(swiglu_handle_t h, const void* W1, const void* W2,
                                      void* P, int64_t K, int64_t N, hipStream_t stream) {
  if (!h || K < 0 || N < 0) return SWIGLU_ERR_INVALID_ARG;
  if (K == 0 || N == 0) return SWIGLU_OK;
  if (!W1 || !W2 || !P) return SWIGLU_ERR_INVALID_ARG;
  if (K > kMaxDim || N > (kMaxDim >> 1)) return SWIGLU_ERR_UNSUPPORTED;
  if (N % 8 != 0 || K % 8 != 0) return SWIGLU_ERR_UNSUPPORTED;
  if (!aligned16(W1) || !aligned16(W2) || !aligned16(P)) return SWIGLU_ERR_UNSUPPORTED;
  const long long wb = 2LL * K * N, pb = 2LL * packed_elems(N, K);
  if (wb >= kMaxBytes || pb >= kMaxBytes) return SWIGLU_ERR_UNSUPPORTED;
  if (overlaps(P, pb, W1, wb) || overlaps(P, pb, W2, wb)) return SWIGLU_ERR_INVALID_ARG;
  swiglu_status_t st = check_device(h);
  if (st != SWIGLU_OK) return st;
  if (launch_pack_frag((const uint16_t*)W1, (const uint16_t*)W2, (uint16_t*)P, (int)N, (int)K,
                       stream, h->cu_count) != hipSuccess)
    return SWIGLU_ERR_LAUNCH;
  return SWIGLU_OK;
}

swiglu_status_t swiglu_forward_fp8(swiglu_handle_t h, const void* A8, const void* W8, void* Y,
                                   int64_t M, int64_t N, int64_t K, float scale_a,
                                   float scale_w1, float scale_w2, swiglu_variant_t variant,
                                   int32_t config_id, hipStream_t stream) {
  if (!h || M < 0 || N < 0 || K < 0) return SWIGLU_ERR_INVALID_ARG;
  const int want = fp8_family((int)variant);
  if (want < 0 || want == VAR_MX || want == VAR_MX_PACKED || want == VAR_MX_SYNC)
    return SWIGLU_ERR_INVALID_ARG;
  int id = config_id;
  if (id >= 0) {
    const KernelConfig* c = config_at(id);
    if (!c || c->variant != want) return SWIGLU_ERR_INVALID_ARG;
  }
  if (M == 0 || N == 0) return SWIGLU_OK;
  if (!Y || (K > 0 && (!A8 || !W8))) return SWIGLU_ERR_INVALID_ARG;
  if (M > kMaxDim || K > kMaxDim || N > (kMaxDim >> 1)) return SWIGLU_ERR_UNSUPPORTED;
  if (N % 8 != 0 || K % 16 != 0) return SWIGLU_ERR_UNSUPPORTED;
  if (!aligned16(Y) || !aligned16(A8) || !aligned16(W8)) return SWIGLU_ERR_UNSUPPORTED;
  const long long ybytes = 2LL * M * N, abytes = M * K;
  const long long wbytes = want == VAR_F8_PACKED ? f8_packed_bytes(N, K) : 2LL * N * K;
  if (ybytes >= kMaxBytes || abytes >= kMaxBytes || wbytes >= kMaxBytes)
    return SWIGLU_ERR_UNSUPPORTED;
  if (K > 0 && (overlaps(Y, ybytes, A8, abytes) || overlaps(Y, ybytes, W8, wbytes)))
    return SWIGLU_ERR_INVALID_ARG;
  swiglu_status_t st = check_device(h);
  if (st != SWIGLU_OK) return st;
  if (id < 0) id = choose(h, want, M, N, K);
  if (id < 0) return SWIGLU_ERR_UNSUPPORTED;
  if (!config_fits(config_at(id), M)) return SWIGLU_ERR_UNSUPPORTED;
  LaunchArgs a;
  a.A = (const uint16_t*)A8;  // byte tensors; the FP8 launchers take them as such
  a.W1 = (const uint16_t*)W8;
  a.W2 = nullptr;
  a.Y = (uint16_t*)Y;
  a.M = (int)M, a.N = (int)N, a.K = (int)K;
  a.ldw = (int)K;
  a.ldy = (int)N;
  a.group_m = 0;
  a.cu_count = h->cu_count;
  a.scale_g = scale_a * scale_w1;
  a.scale_u = scale_a * scale_w2;
  a.stream = stream;
  return launch(h, config_at(id), id, a);
}

}  // extern "C"

namespace {
// MXFP8 forward on W8 in k-major order (want = VAR_MX; a given config may
// also be of the sync order, VAR_MX_SYNC, on the same W8) or in the streaming
// kernel's fragment order (want = VAR_MX_PACKED)
swiglu_status_t forward_mx(swiglu_handle_t h, const void* A8, const void* SA, const void* W8,
                           const void* SW, void* Y, int64_t M, int64_t N, int64_t K, int64_t ks,
                           int32_t config_id, hipStream_t stream, int want) {
  if (!h || M < 0 || N < 0 || K < 0 || ks < 0) return SWIGLU_ERR_INVALID_ARG;
  int id = config_id;
  if (id >= 0) {
    const KernelConfig* c = config_at(id);
    if (!c || (c->variant != want && !(want == VAR_MX && c->variant == VAR_MX_SYNC)))
      return SWIGLU_ERR_INVALID_ARG;
  }
  if (M == 0 || N == 0) return SWIGLU_OK;
  if (!Y || (K > 0 && (!A8 || !W8 || !SA || !SW))) return SWIGLU_ERR_INVALID_ARG;
  if (ks < K / 32) return SWIGLU_ERR_INVALID_ARG;
  if (M > kMaxDim || K > kMaxDim || N > (kMaxDim >> 1) || ks > kMaxDim)
    return SWIGLU_ERR_UNSUPPORTED;
  if (N % 8 != 0 || K % 64 != 0 || ks % 16 != 0) return SWIGLU_ERR_UNSUPPORTED;
  if (!aligned16(Y) || !aligned16(A8) || !aligned16(W8) || !aligned16(SA) || !aligned16(SW))
    return SWIGLU_ERR_UNSUPPORTED;
  const long long ybytes = 2LL * M * N, abytes = M * K;
  const long long wbytes = want == VAR_MX_PACKED ? mx_packed_bytes(N, K) : 2LL * N * K;
  const long long sabytes = M * ks, swbytes = 2LL * N * ks;
  if (ybytes >= kMaxBytes || abytes >= kMaxBytes || wbytes >= kMaxBytes ||
      sabytes >= kMaxBytes || swbytes >= kMaxBytes)
    return SWIGLU_ERR_UNSUPPORTED;
  if (K > 0 && (overlaps(Y, ybytes, A8, abytes) || overlaps(Y, ybytes, W8, wbytes) ||
                overlaps(Y, ybytes, SA, sabytes) || overlaps(Y, ybytes, SW, swbytes)))
    return SWIGLU_ERR_INVALID_ARG;
  swiglu_status_t st = check_device(h);
  if (st != SWIGLU_OK) return st;
  if (id < 0) id = choose(h, want, M, N, K);
  if (id < 0) return SWIGLU_ERR_UNSUPPORTED;
  if (!config_fits(config_at(id), M)) return SWIGLU_ERR_UNSUPPORTED;
  LaunchArgs a;
  a.A = (const uint16_t*)A8;
  a.W1 = (const uint16_t*)W8;
  a.W2 = nullptr;
  a.Y = (uint16_t*)Y;
  a.M = (int)M, a.N = (int)N, a.K = (int)K;
  a.ldw = (int)K;
  a.ldy = (int)N;
  a.group_m = 0;
  a.cu_count = h->cu_count;
  a.scale_g = a.scale_u = 1.0f;
  a.SA = (const uint8_t*)SA;
  a.SW = (const uint8_t*)SW;
  a.ks = (int)ks;
  a.stream = stream;
  return launch(h, config_at(id), id, a);
}

}  // namespace

extern "C" {

swiglu_status_t swiglu_forward_mx(swiglu_handle_t h, const void* A8, const void* SA,
                                  const void* W8, const void* SW, void* Y, int64_t M, int64_t N,
                                  int64_t K, int64_t ks, int32_t config_id, hipStream_t stream) {
  return forward_mx(h, A8, SA, W8, SW, Y, M, N, K, ks, config_id, stream, VAR_MX);
}

// ---- split-K streaming decode ---------------------------------------------------

constexpr int kMaxSplit = 64;  // workgroups per (slab, part) along K

// The split for a decode shape.  Slab parts as in the packed table (whole
// slabs from 1.75 slabs per CU, config 85; half slabs from one per CU, 86;
// quarter slabs below, 87), then K in as many pieces as it takes to give
// every CU a workgroup, each piece keeping at least 16 K steps.  Measured on
// MI355X at M = 16: the split pays only where the parts alone leave CUs idle
// (N = 1184, K = 3584: 10.0 us with the 4 pieces this rule takes, 9.0 with 3,
// 11.6 with one), since
// the handoff adds memory round trips to the last workgroup of each part.
void splitk_plan(long long N, long long K, int cus, int32_t* id, int32_t* S) {
  const long long c = cus > 0 ? cus : 256;
  const long long slabs = packed_slabs(N), steps = packed_steps(K);
  int parts;
  if (4 * slabs >= 7 * c) {
    *id = 85, parts = 1;
  } else if (slabs >= c) {
    *id = 86, parts = 2;
  } else {
    *id = 87, parts = 4;
  }
  const long long units = slabs * parts;
  long long s = (c + units - 1) / units;
  s = std::min<long long>(s, std::max<long long>(1, steps / 16));
  *S = (int32_t)std::max<long long>(1, std::min<long long>(s, kMaxSplit));
}

int64_t swiglu_packed_splitk_workspace_bytes(int64_t N, int64_t K, int32_t ksplit) {
  if (N <= 0 || K < 0 || N > (kMaxDim >> 1) || K > kMaxDim || ksplit < 1 || ksplit > kMaxSplit)
    return 0;
  return splitk_workspace_bytes(packed_slabs(N), ksplit);
}

swiglu_status_t swiglu_packed_splitk_plan(swiglu_handle_t h, int64_t M, int64_t N, int64_t K,
                                          int32_t* config_id, int32_t* ksplit) {
  if (!h || M < 0 || N < 0 || K < 0) return SWIGLU_ERR_INVALID_ARG;
  if (M > 16 || N > (kMaxDim >> 1) || K > kMaxDim) return SWIGLU_ERR_UNSUPPORTED;
  int32_t id, S;
  splitk_plan(N, K, h->cu_count, &id, &S);
  if (config_id) *config_id = id;
  if (ksplit) *ksplit = S;
  return SWIGLU_OK;
}

swiglu_status_t swiglu_forward_packed_splitk(swiglu_handle_t h, const void* A, const void* P,
                                             void* Y, int64_t M, int64_t N, int64_t K,
                                             int32_t config_id, int32_t ksplit, void* workspace,
                                             int64_t workspace_bytes, hipStream_t stream) {
  bool noop = false;
  swiglu_status_t st = check_forward(h, A, P, nullptr, Y, M, N, K, SWIGLU_LAYOUT_PACKED, &noop);
  if (st != SWIGLU_OK) return st;
  if (config_id >= 0) {
    const KernelConfig* c = config_at(config_id);
    if (!c || c->variant != VAR_PACKED_SPLITK) return SWIGLU_ERR_INVALID_ARG;
  }
  if (ksplit > kMaxSplit) return SWIGLU_ERR_UNSUPPORTED;
  if (noop) return SWIGLU_OK;
  if (M > 16) return SWIGLU_ERR_UNSUPPORTED;
  int32_t id = config_id, S = ksplit;
  if (id < 0 || S < 1) {
    int32_t pid, pS;
    splitk_plan(N, K, h->cu_count, &pid, &pS);
    if (id < 0) id = pid;
    if (S < 1) S = pS;
  }
  const long long need = splitk_workspace_bytes(packed_slabs(N), S);
  if (!workspace || workspace_bytes < need) return SWIGLU_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return SWIGLU_ERR_UNSUPPORTED;
  if (overlaps(workspace, need, Y, 2LL * M * N) || overlaps(workspace, need, A, 2LL * M * K) ||
      overlaps(workspace, need, P, 2LL * packed_elems(N, K)))
    return SWIGLU_ERR_INVALID_ARG;
  const KernelConfig* cfg = config_at(id);
  LaunchArgs a;
  a.A = (const uint16_t*)A;
  a.W1 = (const uint16_t*)P;
  a.W2 = nullptr;
  a.Y = (uint16_t*)Y;
  a.M = (int)M, a.N = (int)N, a.K = (int)K;
  a.ldw = 0;
  a.ldy = (int)N;
  a.group_m = 0;
  a.cu_count = h->cu_count;
  a.stream = stream;
  a.ws = workspace;
  a.ksplit = S;
  return launch(h, cfg, id, a);
}

swiglu_status_t swiglu_forward_mx_packed(swiglu_handle_t h, const void* A8, const void* SA,
                                         const void* P8, const void* SW, void* Y, int64_t M,
                                         int64_t N, int64_t K, int64_t ks, int32_t config_id,
                                         hipStream_t stream) {
  return forward_mx(h, A8, SA, P8, SW, Y, M, N, K, ks, config_id, stream, VAR_MX_PACKED);
}

int64_t swiglu_mx_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % 64 != 0 || N > (kMaxDim >> 1) || K > kMaxDim) return 0;
  return mx_packed_bytes(N, K);
}

swiglu_status_t swiglu_pack_mx_fragments(swiglu_handle_t h, const void* W8, void* P8, int64_t K,
                                         int64_t N, hipStream_t stream) {
  if (!h || K < 0 || N < 0) return SWIGLU_ERR_INVALID_ARG;
  if (K == 0 || N == 0) return SWIGLU_OK;
  if (!W8 || !P8) return SWIGLU_ERR_INVALID_ARG;
  if (K > kMaxDim || N > (kMaxDim >> 1)) return SWIGLU_ERR_UNSUPPORTED;
  if (N % 8 != 0 || K % 64 != 0) return SWIGLU_ERR_UNSUPPORTED;
  if (!aligned16(W8) || !aligned16(P8)) return SWIGLU_ERR_UNSUPPORTED;
  const long long wb = 2LL * K * N, pb = mx_packed_bytes(N, K);
  if (wb >= kMaxBytes || pb >= kMaxBytes) return SWIGLU_ERR_UNSUPPORTED;
  if (overlaps(P8, pb, W8, wb)) return SWIGLU_ERR_INVALID_ARG;
  swiglu_status_t st = check_device(h);
  if (st != SWIGLU_OK) return st;
  if (launch_pack_mx_frag((const uint8_t*)W8, (uint8_t*)P8, (int)(2 * N), (int)K, stream,
                          h->cu_count) != hipSuccess)
    return SWIGLU_ERR_LAUNCH;
  return SWIGLU_OK;
}

swiglu_status_t swiglu_quantize_mx(swiglu_handle_t h, const void* X, void* Q, void* S,
                                   int64_t rows, int64_t K, int64_t ks, hipStream_t stream) {
  if (!h || rows < 0 || K < 0 || ks < 0) return SWIGLU_ERR_INVALID_ARG;
  if (rows == 0 || K == 0) return SWIGLU_OK;
  if (!X || !Q || !S || ks < K / 32) return SWIGLU_ERR_INVALID_ARG;
  if (K % 32 != 0 || ks % 16 != 0) return SWIGLU_ERR_UNSUPPORTED;
  if (!aligned16(X) || !aligned16(Q) || !aligned16(S)) return SWIGLU_ERR_UNSUPPORTED;
  if (rows > kMaxDim || K > kMaxDim || ks > kMaxDim || rows * K > (1LL << 40) ||
      rows * ks > (1LL << 40))
    return SWIGLU_ERR_UNSUPPORTED;
  if (overlaps(Q, rows * K, X, 2 * rows * K) || overlaps(S, rows * ks, X, 2 * rows * K) ||
      overlaps(S, rows * ks, Q, rows * K))
    return SWIGLU_ERR_INVALID_ARG;
  swiglu_status_t st = check_device(h);
  if (st != SWIGLU_OK) return st;
  if (launch_quantize_mx((const uint16_t*)X, (uint8_t*)Q, (uint8_t*)S, (int)rows, (int)K,
                         (int)ks, stream, h->cu_count) != hipSuccess)
    return SWIGLU_ERR_LAUNCH;
  return SWIGLU_OK;
}

swiglu_status_t swiglu_pack_kmajor(swiglu_handle_t h, const void* W1, const void* W2, void* Wt,
                                   int64_t K, int64_t N, hipStream_t stream) {
  if (!h || K < 0 || N < 0) return SWIGLU_ERR_INVALID_ARG;
  if (K == 0 || N == 0) return SWIGLU_OK;
  if (!W1 || !W2 || !Wt) return SWIGLU_ERR_INVALID_ARG;
  if (K > kMaxDim || N > (kMaxDim >> 1)) return SWIGLU_ERR_UNSUPPORTED;
  if (N % 8 != 0 || K % 8 != 0) return SWIGLU_ERR_UNSUPPORTED;
  if (!aligned16(W1) || !aligned16(W2) || !aligned16(Wt)) return SWIGLU_ERR_UNSUPPORTED;
  const long long wb = 2LL * K * N;
  if (2 * wb >= kMaxBytes) return SWIGLU_ERR_UNSUPPORTED;
  if (overlaps(Wt, 2 * wb, W1, wb) || overlaps(Wt, 2 * wb, W2, wb)) return SWIGLU_ERR_INVALID_ARG;
  swiglu_status_t st = check_device(h);
  if (st != SWIGLU_OK) return st;
  if (launch_pack_kmajor((const uint16_t*)W1, (const uint16_t*)W2, (uint16_t*)Wt, (int)N, (int)K,
                         stream, h->cu_count) != hipSuccess)
    return SWIGLU_ERR_LAUNCH;
  return SWIGLU_OK;
}

swiglu_status_t swiglu_quantize_fp8(swiglu_handle_t h, const void* X, void* Q, int64_t count,
                                    float inv_scale, hipStream_t stream) {
  if (!h || count < 0) return SWIGLU_ERR_INVALID_ARG;
  if (count == 0) return SWIGLU_OK;
  if (!X || !Q) return SWIGLU_ERR_INVALID_ARG;
  if (count % 16 != 0 || !aligned16(X) || !aligned16(Q)) return SWIGLU_ERR_UNSUPPORTED;
  if (count > (1LL << 40)) return SWIGLU_ERR_UNSUPPORTED;
  if (overlaps(Q, count, X, 2 * count)) return SWIGLU_ERR_INVALID_ARG;
  swiglu_status_t st = check_device(h);
  if (st != SWIGLU_OK) return st;
  if (launch_quantize_f8((const uint16_t*)X, (uint8_t*)Q, (size_t)count, inv_scale, stream,
                         h->cu_count) != hipSuccess)
    return SWIGLU_ERR_LAUNCH;
  return SWIGLU_OK;
}

swiglu_status_t swiglu_pack_fp8(swiglu_handle_t h, const void* W1, const void* W2, void* W8,
                                int64_t K, int64_t N, hipStream_t stream) {
  if (!h || K < 0 || N < 0) return SWIGLU_ERR_INVALID_ARG;
  if (K == 0 || N == 0) return SWIGLU_OK;
  if (!W1 || !W2 || !W8) return SWIGLU_ERR_INVALID_ARG;
  if (K > kMaxDim || N > (kMaxDim >> 1)) return SWIGLU_ERR_UNSUPPORTED;
  if (N % 8 != 0 || K % 16 != 0) return SWIGLU_ERR_UNSUPPORTED;
  if (!aligned16(W1) || !aligned16(W2) || !aligned16(W8)) return SWIGLU_ERR_UNSUPPORTED;
  const long long wb = K * N;
  if (2 * wb >= kMaxBytes) return SWIGLU_ERR_UNSUPPORTED;
  if (overlaps(W8, 2 * wb, W1, wb) || overlaps(W8, 2 * wb, W2, wb)) return SWIGLU_ERR_INVALID_ARG;
  swiglu_status_t st = check_device(h);
  if (st != SWIGLU_OK) return st;
  if (launch_pack_f8((const uint8_t*)W1, (const uint8_t*)W2, (uint8_t*)W8, (int)N, (int)K, stream,
                     h->cu_count) != hipSuccess)
    return SWIGLU_ERR_LAUNCH;
  return SWIGLU_OK;
}

swiglu_status_t swiglu_query_fp8(swiglu_handle_t h, int64_t M, int64_t N, int64_t K,
                                 swiglu_variant_t variant, swiglu_tile_t* tile) {
  if (!h || M < 0 || N < 0 || K < 0) return SWIGLU_ERR_INVALID_ARG;
  const int want = fp8_family((int)variant);
  if (want < 0) return SWIGLU_ERR_INVALID_ARG;
  const int id = choose(h, want, M, N, K);
  if (id < 0) return SWIGLU_ERR_UNSUPPORTED;
  if (tile) fill_tile(id, tile);
  return SWIGLU_OK;
}

swiglu_status_t swiglu_query(swiglu_handle_t h, int64_t M, int64_t N, int64_t K,
                             swiglu_layout_t layout, swiglu_variant_t* chosen,
                             swiglu_tile_t* tile, swiglu_layout_t* recommended_layout) {
  if (!h || M < 0 || N < 0 || K < 0) return SWIGLU_ERR_INVALID_ARG;
  if (layout != SWIGLU_LAYOUT_SEPARATE && layout != SWIGLU_LAYOUT_INTERLEAVED &&
      layout != SWIGLU_LAYOUT_PACKED)
    return SWIGLU_ERR_INVALID_ARG;
  const int want = layout_family((int)layout);
  const int id = choose(h, want, M, N, K);
  if (id < 0) return SWIGLU_ERR_UNSUPPORTED;
  if (chosen) *chosen = (swiglu_variant_t)want;
  if (tile) fill_tile(id, tile);
  if (recommended_layout)
    *recommended_layout = (swiglu_layout_t)recommend_layout(M, N, K, h->cu_count);
  return SWIGLU_OK;
}

swiglu_status_t swiglu_query_unfused(swiglu_handle_t h, int64_t M, int64_t N, int64_t K,
                                     swiglu_tile_t* tile) {
  if (!h || M < 0 || N < 0 || K < 0) return SWIGLU_ERR_INVALID_ARG;
  const int id = choose(h, VAR_GEMM, M, N, K);
  if (id < 0) return SWIGLU_ERR_UNSUPPORTED;
  if (tile) fill_tile(id, tile);
  return SWIGLU_OK;
}

uint64_t swiglu_config_signature(void) { return config_signature(); }

swiglu_status_t swiglu_tuned_check(const char* path, int32_t* n_entries) {
  std::vector<swiglu_tuned_entry> e;
  const swiglu_status_t st = read_tuned(path, &e);
  if (n_entries) *n_entries = st == SWIGLU_OK ? (int32_t)e.size() : 0;
  return st;
}

swiglu_status_t swiglu_create_tuned(swiglu_handle_t* out, int device, const char* path) {
  if (!out) return SWIGLU_ERR_INVALID_ARG;
  *out = nullptr;
  std::vector<swiglu_tuned_entry> e;
  if (path) {
    const swiglu_status_t st = read_tuned(path, &e);
    if (st != SWIGLU_OK) return st;
  }
  swiglu_handle_t h = nullptr;
  const swiglu_status_t st = swiglu_create(&h, device);
  if (st != SWIGLU_OK) return st;
  h->tuned.swap(e);
  *out = h;
  return SWIGLU_OK;
}

int32_t swiglu_config_count(void) { return config_count(); }

swiglu_status_t swiglu_config_info(int32_t config_id, swiglu_tile_t* out) {
  if (!out || !config_at(config_id)) return SWIGLU_ERR_INVALID_ARG;
  fill_tile(config_id, out);
  return SWIGLU_OK;
}

const char* swiglu_status_str(swiglu_status_t s) {
  switch (s) {
    case SWIGLU_OK: return "ok";
    case SWIGLU_ERR_INVALID_ARG: return "invalid argument";
    case SWIGLU_ERR_UNSUPPORTED: return "unsupported shape, alignment or configuration";
    case SWIGLU_ERR_DEVICE: return "no usable gfx950 device";
    case SWIGLU_ERR_LAUNCH: return "kernel launch failed";
    case SWIGLU_ERR_ALLOC: return "host allocation failed";
  }
  return "unknown status";
}

}  // extern "C"
