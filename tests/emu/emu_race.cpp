// LDS ordering check for the CPU emulation: the timing the emulation does not
// have (DMA that lands asynchronously, waves that run concurrently between
// barriers) is modelled from the order of events each thread logs, and every
// LDS access that a GPU could see racing is reported.
//
// The model, per workgroup:
//  * a thread's barrier count is its epoch; waves run in any order inside an
//    epoch, so two accesses of different waves in the same epoch are
//    unordered (one of them a write: a race);
//  * an LDS DMA (buffer_load ... lds) may land at any time from its issue to
//    the s_waitcnt that retires it: wait_vmcnt<N> retires every vector-memory
//    load of the thread except the N most recent (loads complete in order).
//    Global stores are not counted, so the model retires at most what the
//    hardware guarantees.  The compiler's own waits are not seen either: the
//    model may report a race the hardware would not have, never miss one;
//  * a DMA write therefore conflicts with an access of another wave whose
//    epoch lies in [issue epoch, retire epoch], and with an access of its own
//    wave that comes after the issue and before the retiring wait.
// Two DMA writes to the same bytes are not checked against each other (every
// wave writes the zero-fill of a load that has nothing to load into one
// shared junk slot, which is never read).  Also reported: threads of one
// workgroup that pass different numbers of barriers, and a DMA that is still
// in flight when its thread ends.
//
// Plain LDS loads and stores reach this file through the sanitizer-coverage
// load/store callbacks (the kernel translation unit is built with
// -fsanitize-coverage=func,trace-loads,trace-stores); this file itself is
// built without them.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <deque>
#include <string>
#include <vector>

namespace {

enum Kind : uint8_t { EV_READ = 0, EV_WRITE = 1, EV_DMA = 2 };
constexpr uint32_t kOpen = 0xffffffffu;

struct Ev {
  uint32_t off;
  uint16_t len;
  uint8_t kind;
  uint16_t thread;
  uint32_t e0, e1;  // epochs: plain accesses e0 == e1; DMA issue .. retire
  uint32_t i0, i1;  // thread op index (DMA issues, waits, barriers)
};

bool g_on = false;
const uint8_t* g_lds = nullptr;
size_t g_lds_n = 0;
std::vector<Ev> g_ev;
std::deque<int64_t> g_vmq;  // the current thread's vector-memory loads: DMA event or -1
uint32_t g_epoch = 0, g_op = 0;
int g_thread = -1;
std::vector<uint32_t> g_final_epoch;
long g_races = 0;
std::string g_ctx;
struct Range {
  const uint8_t* p;
  size_t n;
};
std::vector<Range> g_globals;  // the launch's global buffers

bool is_global(const uint8_t* b) {
  for (const Range& r : g_globals)
    if (b >= r.p && b < r.p + r.n) return true;
  return false;
}

void race(const char* what, const Ev& a, const Ev* b) {
  ++g_races;
  if (g_races > 12) return;
  fprintf(stderr, "LDS RACE: %s in %s: bytes [%u, %u) thread %u (epoch %u..%u)", what, g_ctx.c_str(),
          a.off, a.off + a.len, a.thread, a.e0, a.e1 == kOpen ? 0u : a.e1);
  if (b)
    fprintf(stderr, " vs bytes [%u, %u) thread %u (epoch %u)", b->off, b->off + b->len, b->thread,
            b->e0);
  fprintf(stderr, "\n");
}

void end_thread() {
  if (g_thread < 0) return;
  for (int64_t e : g_vmq)
    if (e >= 0) g_ev[(size_t)e].e1 = kOpen;  // never retired
  g_vmq.clear();
  g_final_epoch.push_back(g_epoch);
  g_thread = -1;
}

void log_access(const void* p, uint32_t n, uint8_t kind) {
  if (!g_on || g_thread < 0) return;
  const uint8_t* b = (const uint8_t*)p;
  if (g_lds && b >= g_lds && b + n <= g_lds + g_lds_n) {
    g_ev.push_back(Ev{(uint32_t)(b - g_lds), (uint16_t)n, kind, (uint16_t)g_thread, g_epoch, g_epoch,
                      g_op, g_op});
  } else if (kind == EV_READ && is_global(b)) {
    g_vmq.push_back(-1);  // a plain global load occupies a vmcnt slot too
  }
}

bool overlap(const Ev& a, const Ev& b) { return a.off < b.off + b.len && b.off < a.off + a.len; }

}  // namespace

void emu_race_enable(bool on) { g_on = on; }
bool emu_race_enabled() { return g_on; }
void emu_race_global(const void* p, size_t n) { g_globals.push_back(Range{(const uint8_t*)p, n}); }
void emu_race_globals_clear() { g_globals.clear(); }
void emu_race_context(const char* ctx) { g_ctx = ctx; }
long emu_race_count() { return g_races; }
void emu_race_lds(const uint8_t* base, size_t n) { g_lds = base, g_lds_n = n; }

void emu_race_block_begin() {
  g_ev.clear();
  g_final_epoch.clear();
  g_thread = -1;
}
void emu_race_thread(unsigned t) {
  end_thread();
  g_thread = (int)t;
  g_epoch = 0;
  g_op = 0;
}
void emu_race_barrier() {
  ++g_epoch;
  ++g_op;
}
void emu_race_wait(int n) {
  ++g_op;
  while (g_vmq.size() > (size_t)n) {
    const int64_t e = g_vmq.front();
    g_vmq.pop_front();
    if (e >= 0) {
      g_ev[(size_t)e].e1 = g_epoch;
      g_ev[(size_t)e].i1 = g_op;
    }
  }
}
void emu_race_vmop() {
  if (g_on && g_thread >= 0) g_vmq.push_back(-1);
}
void emu_race_dma(uint32_t dst, uint32_t n) {
  if (!g_on || g_thread < 0) return;
  ++g_op;
  g_vmq.push_back((int64_t)g_ev.size());
  g_ev.push_back(Ev{dst, (uint16_t)n, EV_DMA, (uint16_t)g_thread, g_epoch, kOpen, g_op, kOpen});
}
void emu_race_read(const void* p, uint32_t n) { log_access(p, n, EV_READ); }

// Checks one workgroup's log; returns the races found in it.
long emu_race_block_end() {
  end_thread();
  if (!g_on) return 0;
  const long before = g_races;
  for (size_t t = 1; t < g_final_epoch.size(); ++t)
    if (g_final_epoch[t] != g_final_epoch[0]) {
      Ev e{0, 0, EV_READ, (uint16_t)t, g_final_epoch[t], g_final_epoch[0], 0, 0};
      race("threads pass different numbers of barriers", e, nullptr);
      break;
    }
  // events by 16-byte LDS chunk (every access is at most 16 bytes and
  // naturally aligned, so it lies in one chunk)
  const size_t nchunk = g_lds_n / 16 + 1;
  std::vector<std::vector<uint32_t>> dma(nchunk), plain(nchunk);
  for (size_t i = 0; i < g_ev.size(); ++i) {
    const Ev& e = g_ev[i];
    if (e.kind == EV_DMA && e.e1 == kOpen) race("DMA still in flight when its thread ends", e, nullptr);
    (e.kind == EV_DMA ? dma : plain)[e.off / 16].push_back((uint32_t)i);
    if ((e.off + e.len - 1) / 16 != e.off / 16) race("access straddles a 16-byte chunk", e, nullptr);
  }
  for (size_t c = 0; c < nchunk && g_races - before < 12; ++c) {
    std::vector<uint32_t>& pl = plain[c];
    std::sort(pl.begin(), pl.end(), [](uint32_t a, uint32_t b) { return g_ev[a].e0 < g_ev[b].e0; });
    for (uint32_t di : dma[c]) {
      const Ev& d = g_ev[di];
      if (d.e1 == kOpen) continue;
      auto lo = std::lower_bound(pl.begin(), pl.end(), d.e0,
                                 [](uint32_t a, uint32_t e) { return g_ev[a].e0 < e; });
      for (auto it = lo; it != pl.end() && g_ev[*it].e0 <= d.e1; ++it) {
        const Ev& p = g_ev[*it];
        if (!overlap(d, p)) continue;
        const bool same_wave = p.thread / 64 == d.thread / 64;
        if (!same_wave || (d.i0 <= p.i0 && p.i0 < d.i1)) {
          race(p.kind == EV_READ ? "LDS read while a DMA into it may land"
                                 : "LDS write while a DMA into it may land",
               d, &p);
          break;
        }
      }
    }
    // plain accesses of different waves in one epoch, one of them a write
    for (size_t a = 0; a < pl.size(); ++a) {
      const Ev& x = g_ev[pl[a]];
      for (size_t b = a + 1; b < pl.size() && g_ev[pl[b]].e0 == x.e0; ++b) {
        const Ev& y = g_ev[pl[b]];
        if ((x.kind == EV_WRITE || y.kind == EV_WRITE) && x.thread / 64 != y.thread / 64 &&
            overlap(x, y)) {
          race("LDS accesses of two waves between the same barriers", x, &y);
          break;
        }
      }
    }
  }
  return g_races - before;
}

// sanitizer-coverage callbacks: every load and store of the instrumented
// kernel translation unit
extern "C" {
void __sanitizer_cov_load1(uint8_t* p) { log_access(p, 1, EV_READ); }
void __sanitizer_cov_load2(uint16_t* p) { log_access(p, 2, EV_READ); }
void __sanitizer_cov_load4(uint32_t* p) { log_access(p, 4, EV_READ); }
void __sanitizer_cov_load8(uint64_t* p) { log_access(p, 8, EV_READ); }
void __sanitizer_cov_load16(__int128* p) { log_access(p, 16, EV_READ); }
void __sanitizer_cov_store1(uint8_t* p) { log_access(p, 1, EV_WRITE); }
void __sanitizer_cov_store2(uint16_t* p) { log_access(p, 2, EV_WRITE); }
void __sanitizer_cov_store4(uint32_t* p) { log_access(p, 4, EV_WRITE); }
void __sanitizer_cov_store8(uint64_t* p) { log_access(p, 8, EV_WRITE); }
void __sanitizer_cov_store16(__int128* p) { log_access(p, 16, EV_WRITE); }
}

void emu_copy(void* d, const void* s, size_t n) { memcpy(d, s, n); }
// sink for the operands of the emulated matrix products (keeps their loads)
void emu_use(const void*, size_t) {}
void emu_zero(void* d, size_t n) { memset(d, 0, n); }
