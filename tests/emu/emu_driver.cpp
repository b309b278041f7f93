// CPU bounds emulation of every kernel configuration: the kernel source is
// compiled for the host against a stand-in device header (swiglu_device.hpp
// in this directory), each workgroup's threads are run one after another
// through the real launch functions, and every LDS offset, DMA source and
// direct global load is checked against the buffers actually allocated (the
// build adds AddressSanitizer for the plain pointer accesses: LDS staging,
// global stores).  The threads run one after another, so the data is not
// meaningful; where each access goes is checked, and (emu_race.cpp) whether
// the barriers and DMA waits order every LDS access as a GPU needs.
//
// usage: emu_driver [cfg ...]          all shapes for the listed configs (default: all)
//        emu_driver --shape M N K cfg  one shape
//        --last-blocks B               only the last B workgroups of each launch
//        --no-races                    bounds only (no LDS ordering check)
//        --race-blocks B               the ordering check on the last B workgroups only
//        --ksplit S                    pieces of K for the split-K streaming configs (3)
//        --plant P                     switch on planted mistake P (build.py)
#include <stdio.h>
#include <stdlib.h>

#include <string>
#include <vector>

#include "swiglu_kernels_emu.cpp"

dim3 threadIdx, blockIdx, gridDim, blockDim;
long g_emu_last_blocks = 0;
long g_emu_race_errors = 0;
long g_emu_race_blocks = 0;
int g_emu_ksplit = 3;  // pieces of K for the split-K streaming configs
int g_emu_plant = 0;

// the LDS ordering check (emu_race.cpp)
void emu_race_context(const char* ctx);
void emu_race_lds(const uint8_t* base, size_t n);
void emu_race_global(const void* p, size_t n);
void emu_race_globals_clear();

namespace {
struct Alloc {
  const uint8_t* p;
  size_t n;
  const char* name;
};
std::vector<Alloc> g_allocs;
uint8_t* g_lds = nullptr;
size_t g_lds_size = 0;
long g_errors = 0;
long g_lds_checks = 0, g_global_checks = 0, g_threads = 0;
std::string g_ctx;

void report(const char* what, const void* p, size_t n) {
  if (g_errors < 20)
    fprintf(stderr, "OUT OF BOUNDS: %s (%zu bytes at %p) in %s, block (%u,%u) thread %u\n", what,
            n, p, g_ctx.c_str(), blockIdx.x, blockIdx.y, threadIdx.x);
  ++g_errors;
}
}  // namespace

uint8_t* emu_lds(size_t bytes) {
  if (bytes != g_lds_size || !g_lds) {
    free(g_lds);
    g_lds = (uint8_t*)malloc(bytes ? bytes : 1);
    memset(g_lds, 0, bytes);
    g_lds_size = bytes;
    emu_race_lds(g_lds, bytes);
  }
  return g_lds;
}
uint8_t* emu_lds_base() { return g_lds; }
void emu_barrier() { emu_race_barrier(); }
void emu_check_lds(uint32_t off, size_t n, const char* what) {
  ++g_lds_checks;
  if (!g_lds || (size_t)off + n > g_lds_size) report(what, g_lds ? g_lds + off : nullptr, n);
}
void emu_check_global(const void* p, size_t n, const char* what) {
  ++g_global_checks;
  const uint8_t* b = (const uint8_t*)p;
  if (b)
    for (const Alloc& a : g_allocs)
      if (b >= a.p && b + n <= a.p + a.n) return;
  report(what, p, n);
}

namespace {
uint16_t* alloc16(size_t elems, const char* name) {
  const size_t n = elems * 2;
  uint16_t* p = (uint16_t*)malloc(n ? n : 1);
  memset(p, 0, n);
  g_allocs.push_back({(const uint8_t*)p, n, name});
  emu_race_global(p, n);
  return p;
}
void free_all() {
  for (const Alloc& a : g_allocs) free((void*)a.p);
  g_allocs.clear();
  emu_race_globals_clear();
}

// one configuration on one shape, through the same LaunchArgs the C ABI builds
bool run_config(int id, int M, int N, int K) {
  using namespace swiglu;
  const KernelConfig* c = config_at(id);
  if (!c) return false;
  char buf[160];
  snprintf(buf, sizeof buf, "config %d (variant %d family %d %dx%d) shape M=%d N=%d K=%d", id,
           c->variant, c->family, c->bm, c->bn, M, N, K);
  g_ctx = buf;
  emu_race_context(buf);
  const long before = g_errors + g_emu_race_errors;
  const long l0 = g_lds_checks, g0 = g_global_checks;
  LaunchArgs a{};
  a.M = M, a.N = N, a.K = K;
  if (c->variant == VAR_PACKED_SPLITK && M > 16) a.M = M = 16;
  a.A = alloc16((size_t)M * K, "A");
  if (c->variant == VAR_INTERLEAVE) {
    a.W1 = alloc16((size_t)K * 2 * N, "W_fused");
    a.W2 = nullptr;
    a.ldw = 2 * N;
  } else if (c->variant == VAR_PACKED || c->variant == VAR_PACKED_SPLITK) {
    a.W1 = alloc16((size_t)packed_elems(N, K), "P");  // fragment-ordered W_fused
    a.W2 = nullptr;
    a.ldw = 0;
    if (c->variant == VAR_PACKED_SPLITK) {
      // decode rows only; the workspace zeroed as the API requires
      if (M > 16) a.M = M = 16;
      a.ksplit = g_emu_ksplit;
      a.ws = alloc16((size_t)splitk_workspace_bytes(packed_slabs(N), a.ksplit) / 2, "splitk ws");
    }
  } else if (c->variant == VAR_SYNC) {
    a.W1 = alloc16((size_t)K * N, "W1");
    a.W2 = alloc16((size_t)K * N, "W2");
    a.ldw = N;
  } else {
    a.W1 = alloc16((size_t)K * N, "W");
    a.W2 = nullptr;
    a.ldw = N;
  }
  if (c->variant == VAR_F8 || c->variant == VAR_F8_SYNC || c->variant == VAR_MX ||
      c->variant == VAR_MX_SYNC || c->variant == VAR_F8_PACKED || c->variant == VAR_MX_PACKED) {
    // byte tensors: A8 [M, K], W8 [2N, K] (or its fragment order P8); MX
    // scales SA [M, ks], SW [2N, ks]
    a.A = alloc16(((size_t)M * K + 1) / 2, "A8");
    a.W1 = c->variant == VAR_F8_PACKED   ? alloc16((size_t)f8_packed_bytes(N, K) / 2, "P8")
           : c->variant == VAR_MX_PACKED ? alloc16((size_t)mx_packed_bytes(N, K) / 2, "P8mx")
                                         : alloc16((size_t)N * K, "W8");
    a.ldw = K;
    a.scale_g = a.scale_u = 1.0f;
    if (c->variant == VAR_MX || c->variant == VAR_MX_SYNC || c->variant == VAR_MX_PACKED) {
      a.ks = (K / 32 + 15) / 16 * 16;
      a.SA = (const uint8_t*)alloc16(((size_t)M * a.ks + 1) / 2, "SA");
      a.SW = (const uint8_t*)alloc16((size_t)N * a.ks, "SW");
    }
  }
  a.Y = alloc16((size_t)M * N, "Y");
  a.ldy = N;
  a.group_m = 0;
  a.cu_count = 256;
  a.stream = nullptr;
  const hipError_t e = c->launch(a);
  if (c->variant == VAR_PACKED_SPLITK && e == hipSuccess && g_emu_last_blocks == 0) {
    // every (slab, part) counter is back at zero once the last piece is done
    // (when every workgroup of the launch ran)
    const uint32_t* cnt = (const uint32_t*)a.ws;
    for (long long i = 0; i < packed_slabs(N) * 4; ++i)
      if (cnt[i] != 0) {
        fprintf(stderr, "split-K counter %lld left at %u in %s\n", i, cnt[i], g_ctx.c_str());
        ++g_errors;
        break;
      }
  }
  free_all();
  if (e != hipSuccess) fprintf(stderr, "launch refused: %s\n", g_ctx.c_str());
  const bool ok = g_errors + g_emu_race_errors == before;
  printf("%s: %s (%ld LDS accesses, %ld global reads checked)\n", g_ctx.c_str(),
         ok ? "ok" : "OUT OF BOUNDS OR LDS RACE", g_lds_checks - l0, g_global_checks - g0);
  return ok;
}

bool run_elementwise(size_t n) {
  using namespace swiglu;
  g_ctx = "gate/pack n=" + std::to_string(n);
  emu_race_context(g_ctx.c_str());
  const long before = g_errors + g_emu_race_errors;
  uint16_t* g = alloc16(n, "G");
  uint16_t* u = alloc16(n, "U");
  uint16_t* y = alloc16(n, "Y");
  launch_gate(g, u, y, n, nullptr, 256);
  uint16_t* wf = alloc16(2 * n, "WF");
  launch_pack(g, u, wf, n, nullptr, 256);
  free_all();
  // FP8 quantisation (n bf16 -> n bytes) and the k-major pack of two [K, N]
  // byte matrices (K = 16 rows, N = n / 16 columns)
  uint16_t* x = alloc16(n, "X");
  uint8_t* q = (uint8_t*)alloc16((n + 1) / 2, "Q");
  launch_quantize_f8(x, q, n, 1.0f, nullptr, 256);
  const int K = 16, N = (int)(n / 16);
  uint8_t* w1 = (uint8_t*)alloc16((size_t)K * N / 2, "W1_8");
  uint8_t* w2 = (uint8_t*)alloc16((size_t)K * N / 2, "W2_8");
  uint8_t* w8 = (uint8_t*)alloc16((size_t)K * N, "W8");
  launch_pack_f8(w1, w2, w8, N, K, nullptr, 256);
  free_all();
  // fragment-ordered W8 from W8 [R, 144] (R = n / 144 rounded down to a
  // multiple of 16: a partial step of 128 k)
  {
    const int Kp8 = 144, Rp8 = (int)(n / 144) / 16 * 16;
    if (Rp8 > 0) {
      uint8_t* w8s = (uint8_t*)alloc16((size_t)Rp8 * Kp8 / 2, "W8s");
      uint8_t* p8 = (uint8_t*)alloc16((size_t)f8_packed_bytes(Rp8 / 2, Kp8) / 2, "P8s");
      launch_pack_f8_frag(w8s, p8, Rp8, Kp8, nullptr, 256);
      free_all();
    }
    // MX fragment order from W8 [R, 128] (R = n / 128 rounded down to a
    // multiple of 8: a partial block of 32 rows)
    const int Kmx = 128, Rmx = (int)(n / 128) / 8 * 8;
    if (Rmx > 0) {
      uint8_t* w8m = (uint8_t*)alloc16((size_t)Rmx * Kmx / 2, "W8m");
      uint8_t* pm = (uint8_t*)alloc16((size_t)mx_packed_bytes(Rmx / 2, Kmx) / 2, "P8m");
      launch_pack_mx_frag(w8m, pm, Rmx, Kmx, nullptr, 256);
      free_all();
    }
  }
  // MX quantisation of rows of K = 96 (scale stride 16), and the bf16 k-major pack
  {
    const int Kq = 96, ksq = 16, rows = (int)(n / Kq);
    uint16_t* xq = alloc16((size_t)rows * Kq, "Xmx");
    uint8_t* qq = (uint8_t*)alloc16((size_t)rows * Kq / 2, "Qmx");
    uint8_t* sq = (uint8_t*)alloc16((size_t)rows * ksq / 2, "Smx");
    launch_quantize_mx(xq, qq, sq, rows, Kq, ksq, nullptr, 256);
    const int Kp = 16, Np = (int)(n / 16);
    uint16_t* p1 = alloc16((size_t)Kp * Np, "W1bf");
    uint16_t* p2 = alloc16((size_t)Kp * Np, "W2bf");
    uint16_t* pt = alloc16((size_t)2 * Kp * Np, "Wt");
    launch_pack_kmajor(p1, p2, pt, Np, Kp, nullptr, 256);
    free_all();
  }
  // fragment-ordered W_fused from [K, N] weights (K = 40, N = n / 40 rounded
  // down to a multiple of 8: ragged slabs and steps)
  {
    const int Kf = 40, Nf = (int)(n / 40) / 8 * 8;
    if (Nf > 0) {
      uint16_t* f1 = alloc16((size_t)Kf * Nf, "W1f");
      uint16_t* f2 = alloc16((size_t)Kf * Nf, "W2f");
      uint16_t* pf = alloc16((size_t)packed_elems(Nf, Kf), "Pf");
      launch_pack_frag(f1, f2, pf, Nf, Kf, nullptr, 256);
      free_all();
    }
  }
  const bool ok = g_errors + g_emu_race_errors == before;
  printf("%s: %s\n", g_ctx.c_str(), ok ? "ok" : "OUT OF BOUNDS OR LDS RACE");
  return ok;
}
}  // namespace

int main(int argc, char** argv) {
  using namespace swiglu;
  std::vector<int> ids;
  int shape[3] = {0, 0, 0};
  bool one_shape = false, races = true;
  for (int i = 1; i < argc; ++i) {
    if (std::string(argv[i]) == "--no-races") {
      races = false;
    } else if (std::string(argv[i]) == "--ksplit" && i + 1 < argc) {
      g_emu_ksplit = atoi(argv[++i]);
    } else if (std::string(argv[i]) == "--race-blocks" && i + 1 < argc) {
      g_emu_race_blocks = atol(argv[++i]);
    } else if (std::string(argv[i]) == "--plant" && i + 1 < argc) {
      g_emu_plant = atoi(argv[++i]);
    } else if (std::string(argv[i]) == "--last-blocks" && i + 1 < argc) {
      g_emu_last_blocks = atol(argv[++i]);
    } else if (std::string(argv[i]) == "--shape" && i + 3 < argc) {
      shape[0] = atoi(argv[i + 1]), shape[1] = atoi(argv[i + 2]), shape[2] = atoi(argv[i + 3]);
      one_shape = true;
      i += 3;
    } else {
      ids.push_back(atoi(argv[i]));
    }
  }
  emu_race_enable(races);
  if (ids.empty())
    for (int i = 0; i < config_count(); ++i) ids.push_back(i);
  // the GPU parity shapes (ragged tails in every dimension) and K = 0
  const int shapes[][3] = {{300, 264, 200}, {37, 136, 520}, {1, 8, 8}, {129, 520, 96}, {40, 72, 0}};
  // FP8 tiles need K % 16 == 0: the same shapes with K rounded up to 16
  const int shapes_f8[][3] = {{300, 264, 208}, {37, 136, 528}, {1, 8, 16}, {129, 520, 96}, {40, 72, 0}};
  // MXFP8 tiles need K % 64 == 0
  const int shapes_mx[][3] = {{300, 264, 256}, {37, 136, 576}, {1, 8, 64}, {129, 520, 128}, {40, 72, 0}};
  for (int id : ids) {
    if (one_shape) {
      run_config(id, shape[0], shape[1], shape[2]);
    } else {
      if (config_at(id) && (config_at(id)->variant == VAR_MX || config_at(id)->variant == VAR_MX_SYNC ||
                            config_at(id)->variant == VAR_MX_PACKED))
        for (const auto& s : shapes_mx) run_config(id, s[0], s[1], s[2]);
      else if (config_at(id) && (config_at(id)->variant == VAR_F8 || config_at(id)->variant == VAR_F8_SYNC ||
                                 config_at(id)->variant == VAR_F8_PACKED))
        for (const auto& s : shapes_f8) run_config(id, s[0], s[1], s[2]);
      else
        for (const auto& s : shapes) run_config(id, s[0], s[1], s[2]);
    }
  }
  if (!one_shape) {
    run_elementwise(8);
    run_elementwise(200 * 264);
  }
  printf("errors: %ld\n", g_errors + g_emu_race_errors);
  return g_errors + g_emu_race_errors ? 1 : 0;
}
