// Fiber scheduler, wavefront collectives and guarded allocations of the host
// emulator (see include/emu_runtime.h).  x86-64 Linux only.
#include <signal.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <sys/mman.h>
#include <unistd.h>

#include <algorithm>
#include <cmath>
#include <deque>
#include <map>
#include <random>
#include <vector>

#include "hip/hip_runtime.h"

// Saves the callee-saved registers and the stack pointer of the running
// context into *save_sp and resumes the context whose stack pointer is new_sp.
extern "C" void emu_ctx_switch(void** save_sp, void* new_sp);
asm(R"(
  .text
  .globl emu_ctx_switch
  .type emu_ctx_switch,@function
emu_ctx_switch:
  pushq %rbp
  pushq %rbx
  pushq %r12
  pushq %r13
  pushq %r14
  pushq %r15
  movq %rsp, (%rdi)
  movq %rsi, %rsp
  popq %r15
  popq %r14
  popq %r13
  popq %r12
  popq %rbx
  popq %rbp
  ret
  .size emu_ctx_switch, .-emu_ctx_switch
)");

namespace emu {

dim3* g_tid = nullptr;
dim3 g_bid, g_bdim, g_gdim;

namespace {

enum State { READY, AT_WAVE_OP, AT_BARRIER, DONE };

struct Lane {
  void* sp = nullptr;
  char* stack = nullptr;  // lowest address of the usable stack
  dim3 tid;
  int wave = 0, lane = 0;
  State st = DONE;
  WaveFn op = nullptr;
  LaneIO io;
};

constexpr size_t kStackBytes = 512 * 1024;
constexpr size_t kPage = 4096;

// One direct-to-LDS load instruction of a wave that has not landed yet.
struct DmaOp {
  char* dst;                 // LDS address of lane 0's 16 bytes
  const char* src[kWave];    // global source of each lane's 16 bytes
  uint64_t live;
};

struct Wave {
  int live = 0;     // lanes not finished
  int arrived = 0;  // lanes waiting at the current collective
  WaveFn fn = nullptr;
  std::deque<DmaOp> dma;  // issued, not yet landed (oldest first)
};

std::vector<Lane> g_lanes;
std::vector<Wave> g_waves;
std::vector<int> g_ready;  // lanes that can run
int g_live = 0;            // work-items of the block not finished
int g_at_barrier = 0;
void* g_sched_sp = nullptr;
Lane* g_cur = nullptr;
const std::function<void()>* g_body = nullptr;
int g_op_wave = -1;  // wave whose collective is being computed
std::mt19937_64 g_rng(1);
int g_cus = 8;
unsigned long long g_wave_ops = 0, g_barriers = 0, g_blocks = 0;

void lane_entry() {
  (*g_body)();
  g_cur->st = DONE;
  emu_ctx_switch(&g_cur->sp, g_sched_sp);
  abort();  // a finished fiber is never resumed
}

void ensure_lanes(size_t n) {
  while (g_lanes.size() < n) {
    // one guard page below each stack catches overflows
    char* m = (char*)mmap(nullptr, kStackBytes + kPage, PROT_READ | PROT_WRITE,
                          MAP_PRIVATE | MAP_ANONYMOUS, -1, 0);
    if (m == MAP_FAILED) fail("cannot map a fiber stack");
    mprotect(m, kPage, PROT_NONE);
    g_lanes.emplace_back();
    g_lanes.back().stack = m + kPage;
  }
}

void start_lane(Lane& L) {
  uintptr_t top = ((uintptr_t)(L.stack + kStackBytes)) & ~(uintptr_t)15;
  uint64_t* sp = (uint64_t*)top;
  *--sp = 0;                                 // return address of lane_entry (never used)
  *--sp = (uint64_t)(uintptr_t)&lane_entry;  // taken by the switch's ret
  for (int i = 0; i < 6; ++i) *--sp = 0;     // rbp rbx r12 r13 r14 r15
  L.sp = sp;
  L.st = READY;
}

void yield_to_scheduler() { emu_ctx_switch(&g_cur->sp, g_sched_sp); }

// Computes wave w's collective if every live lane of the wave has reached it.
void complete_wave(int w, int nlanes) {
  Wave& W = g_waves[w];
  if (W.arrived == 0 || W.arrived < W.live) return;
  const int l0 = w * kWave;
  const int n = nlanes - l0 < kWave ? nlanes - l0 : kWave;
  uint64_t live = 0;
  LaneIO* io[kWave] = {};
  for (int l = 0; l < n; ++l) {
    Lane& L = g_lanes[l0 + l];
    if (L.st != AT_WAVE_OP) continue;
    live |= 1ull << l;
    io[l] = &L.io;
  }
  g_op_wave = w;
  W.fn(live, io);
  g_op_wave = -1;
  ++g_wave_ops;
  for (int l = 0; l < n; ++l)
    if (live >> l & 1) {
      g_lanes[l0 + l].st = READY;
      g_ready.push_back(l0 + l);
    }
  W.arrived = 0;
  W.fn = nullptr;
}

void release_barrier(int nlanes) {
  if (g_live == 0 || g_at_barrier < g_live) return;
  for (int i = 0; i < nlanes; ++i)
    if (g_lanes[i].st == AT_BARRIER) {
      g_lanes[i].st = READY;
      g_ready.push_back(i);
    }
  g_at_barrier = 0;
  ++g_barriers;
}

void run_block(int nlanes) {
  ensure_lanes((size_t)nlanes);
  const int nwaves = (nlanes + kWave - 1) / kWave;
  g_waves.assign((size_t)nwaves, Wave());
  g_ready.clear();
  for (int i = 0; i < nlanes; ++i) {
    Lane& L = g_lanes[i];
    L.tid = dim3(i % g_bdim.x, (i / g_bdim.x) % g_bdim.y, i / (g_bdim.x * g_bdim.y));
    L.wave = i / kWave;
    L.lane = i % kWave;
    L.op = nullptr;
    start_lane(L);
    g_waves[L.wave].live++;
    g_ready.push_back(i);
  }
  g_live = nlanes;
  g_at_barrier = 0;
  while (!g_ready.empty()) {
    const size_t k = g_rng() % g_ready.size();
    const int id = g_ready[k];
    g_ready[k] = g_ready.back();
    g_ready.pop_back();
    Lane& L = g_lanes[id];
    Wave& W = g_waves[L.wave];
    g_cur = &L;
    g_tid = &L.tid;
    emu_ctx_switch(&g_sched_sp, L.sp);
    g_cur = nullptr;
    switch (L.st) {
      case AT_WAVE_OP:
        if (W.arrived > 0 && W.fn != L.op) fail("lanes of one wave reached different collectives");
        W.fn = L.op;
        W.arrived++;
        complete_wave(L.wave, nlanes);
        break;
      case AT_BARRIER:
        if (W.arrived > 0) fail("some lanes of a wave wait at a collective, others at a barrier");
        g_at_barrier++;
        release_barrier(nlanes);
        break;
      case DONE:
        W.live--;
        g_live--;
        // lanes that finished early are inactive in later collectives and barriers
        complete_wave(L.wave, nlanes);
        release_barrier(nlanes);
        break;
      default:
        fail("fiber yielded in an unexpected state");
    }
  }
  if (g_live != 0)
    fail("workgroup cannot make progress: a wave waits at a collective that some of its "
         "lanes never reach, or some work-items wait at a barrier others never reach");
  // loads still in flight when the workgroup ends write LDS nobody reads again
  for (Wave& W : g_waves) W.dma.clear();
}

// Lands the oldest direct-to-LDS loads of wave W until at most `keep` remain.
void land_dma(Wave& W, size_t keep) {
  while (W.dma.size() > keep) {
    const DmaOp& op = W.dma.front();
    for (int l = 0; l < kWave; ++l)
      if (op.live >> l & 1) memcpy(op.dst + 16 * l, op.src[l], 16);
    W.dma.pop_front();
  }
}

}  // namespace

void fail(const char* msg) {
  fprintf(stderr, "emulator: %s (block %u,%u,%u)\n", msg, g_bid.x, g_bid.y, g_bid.z);
  fflush(stderr);
  abort();
}

int lane_id() { return g_cur->lane; }

void wave_op(WaveFn fn, const void* in, size_t nin, void* out, size_t nout) {
  Lane& L = *g_cur;
  if (nin > sizeof L.io.in || nout > sizeof L.io.out) fail("wave collective operands too large");
  memcpy(L.io.in, in, nin);
  L.op = fn;
  L.st = AT_WAVE_OP;
  yield_to_scheduler();
  memcpy(out, L.io.out, nout);
}

void block_barrier() {
  g_cur->st = AT_BARRIER;
  yield_to_scheduler();
}

void run_grid(dim3 grid, dim3 block, const std::function<void()>& body) {
  if (g_cur) fail("kernel launched from inside a kernel");
  const long n = (long)block.x * block.y * block.z;
  if (n < 1 || n > 1024) fail("workgroup size must be 1..1024");
  if (grid.x < 1 || grid.y < 1 || grid.z < 1) fail("empty grid");
  g_bdim = block;
  g_gdim = grid;
  g_body = &body;
  for (uint32_t z = 0; z < grid.z; ++z)
    for (uint32_t y = 0; y < grid.y; ++y)
      for (uint32_t x = 0; x < grid.x; ++x) {
        g_bid = dim3(x, y, z);
        run_block((int)n);
        ++g_blocks;
      }
  g_body = nullptr;
}

// ------------------------------------------------------------------ collectives

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

void op_mfma_16x16x32_bf16(uint64_t live, LaneIO* const* io) {
  if (live != ~0ull) fail("MFMA needs all 64 lanes");
  double A[16][32], B[32][16];
  for (int l = 0; l < kWave; ++l) {
    const int i = l & 15, g = l >> 4;
    uint16_t a[8], b[8];
    memcpy(a, io[l]->in, 16);
    memcpy(b, io[l]->in + 16, 16);
    for (int j = 0; j < 8; ++j) {
      A[i][8 * g + j] = bf16_to_f32(a[j]);
      B[8 * g + j][i] = bf16_to_f32(b[j]);
    }
  }
  for (int l = 0; l < kWave; ++l) {
    const int n = l & 15, g = l >> 4;
    float c[4], d[4];
    memcpy(c, io[l]->in + 32, 16);
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      double s = 0;
      for (int k = 0; k < 32; ++k) s += A[m][k] * B[k][n];
      d[r] = (float)((double)c[r] + s);
    }
    memcpy(io[l]->out, d, 16);
  }
}

void op_tr16_b64(uint64_t live, LaneIO* const* io) {
  if (live != ~0ull) fail("transposing LDS read needs all 64 lanes");
  const uint16_t* src[kWave];
  for (int l = 0; l < kWave; ++l) {
    memcpy(&src[l], io[l]->in, sizeof(void*));
    if ((uintptr_t)src[l] & 7) fail("transposing LDS read: address not 8-byte aligned");
  }
  for (int l = 0; l < kWave; ++l) {
    const int g = l >> 4, i = l & 15;
    uint16_t r[4];
    for (int k = 0; k < 4; ++k) r[k] = src[16 * g + 4 * k + (i >> 2)][i & 3];
    memcpy(io[l]->out, r, 8);
  }
}

// OCP e4m3 value of a code (NaN for 0x7F / 0xFF)
static double e4m3_value(unsigned char c) {
  const int e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
  return (c & 0x80) ? -v : v;
}

double e4m3_to_double(unsigned char c) { return e4m3_value(c); }

// fp32 -> e4m3 by search over the codes (nearest, ties to the even code;
// magnitudes past 448 saturate; NaN -> 0x7F)
unsigned char f32_to_e4m3_rne(float x) {
  if (std::isnan(x)) return 0x7f;
  const double a = std::min(std::fabs((double)x), 448.0);
  int best = 0;
  double bd = 1e300;
  for (int c = 0; c <= 0x7e; ++c) {
    const double d = std::fabs(e4m3_value((unsigned char)c) - a);
    if (d < bd || (d == bd && (c & 1) == 0)) {
      bd = d;
      best = c;
    }
  }
  return (unsigned char)(best | (std::signbit(x) ? 0x80 : 0));
}

void op_mfma_16x16x32_fp8(uint64_t live, LaneIO* const* io) {
  if (live != ~0ull) fail("MFMA needs all 64 lanes");
  double A[16][32], B[32][16];
  for (int l = 0; l < kWave; ++l) {
    const int i = l & 15, g = l >> 4;
    unsigned char a[8], b[8];
    memcpy(a, io[l]->in, 8);
    memcpy(b, io[l]->in + 8, 8);
    for (int j = 0; j < 8; ++j) {
      A[i][8 * g + j] = e4m3_value(a[j]);
      B[8 * g + j][i] = e4m3_value(b[j]);
    }
  }
  for (int l = 0; l < kWave; ++l) {
    const int n = l & 15, g = l >> 4;
    float c[4], d[4];
    memcpy(c, io[l]->in + 16, 16);
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      double s = 0;
      for (int k = 0; k < 32; ++k) s += A[m][k] * B[k][n];
      d[r] = (float)((double)c[r] + s);
    }
    memcpy(io[l]->out, d, 16);
  }
}

void op_mfma_16x16x128_f8(uint64_t live, LaneIO* const* io) {
  if (live != ~0ull) fail("MFMA needs all 64 lanes");
  static double A[16][128], B[128][16];
  for (int l = 0; l < kWave; ++l) {
    const int i = l & 15, g = l >> 4;
    unsigned char a[32], b[32];
    memcpy(a, io[l]->in, 32);
    memcpy(b, io[l]->in + 32, 32);
    for (int j = 0; j < 32; ++j) {
      A[i][32 * g + j] = e4m3_value(a[j]);
      B[32 * g + j][i] = e4m3_value(b[j]);
    }
  }
  for (int l = 0; l < kWave; ++l) {
    const int n = l & 15, g = l >> 4;
    float c[4], d[4];
    memcpy(c, io[l]->in + 64, 16);
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      double s = 0;
      for (int k = 0; k < 128; ++k) s += A[m][k] * B[k][n];
      d[r] = (float)((double)c[r] + s);
    }
    memcpy(io[l]->out, d, 16);
  }
}

void op_tr8_b64(uint64_t live, LaneIO* const* io) {
  if (live != ~0ull) fail("transposing LDS read needs all 64 lanes");
  const unsigned char* src[kWave];
  for (int l = 0; l < kWave; ++l) {
    memcpy(&src[l], io[l]->in, sizeof(void*));
    if ((uintptr_t)src[l] & 7) fail("transposing LDS read: address not 8-byte aligned");
  }
  for (int l = 0; l < kWave; ++l) {
    const int g = l >> 4, i = l & 15;
    unsigned char r[8];
    for (int k = 0; k < 8; ++k) r[k] = src[16 * g + 2 * k + (i >> 3)][i & 7];
    memcpy(io[l]->out, r, 8);
  }
}

void op_gather(uint64_t live, LaneIO* const* io) {
  for (int l = 0; l < kWave; ++l) {
    if (!(live >> l & 1)) continue;
    int src;
    memcpy(&src, io[l]->in + 8, 4);
    if (src < 0 || src >= kWave || !(live >> src & 1)) fail("shuffle from a lane that is not live");
    memcpy(io[l]->out, io[src]->in, 8);
  }
}

void op_ballot(uint64_t live, LaneIO* const* io) {
  unsigned long long m = 0;
  for (int l = 0; l < kWave; ++l) {
    if (!(live >> l & 1)) continue;
    int p;
    memcpy(&p, io[l]->in, 4);
    if (p) m |= 1ull << l;
  }
  for (int l = 0; l < kWave; ++l)
    if (live >> l & 1) memcpy(io[l]->out, &m, 8);
}

void op_first(uint64_t live, LaneIO* const* io) {
  const int f = __builtin_ctzll(live);
  for (int l = 0; l < kWave; ++l)
    if (live >> l & 1) memcpy(io[l]->out, io[f]->in, 4);
}

// Direct-to-LDS load: queued; the loads of a wave land in issue order, mostly
// as late as the s_waitcnt that requires them (so a wait that is too weak shows
// up as stale LDS data), sometimes right after they are issued (so a load into
// a buffer that is still being read shows up too).
void op_dma16(uint64_t live, LaneIO* const* io) {
  Wave& W = g_waves[g_op_wave];
  DmaOp op;
  op.live = live;
  op.dst = nullptr;
  for (int l = 0; l < kWave; ++l) {
    op.src[l] = nullptr;
    if (!(live >> l & 1)) continue;
    char* dst;
    memcpy(&op.src[l], io[l]->in, sizeof(void*));
    memcpy(&dst, io[l]->in + 8, sizeof(void*));
    if (op.dst && dst != op.dst) fail("direct-to-LDS load: LDS base differs between lanes");
    op.dst = dst;
  }
  W.dma.push_back(op);
  if (g_rng() % 8 == 0) land_dma(W, g_rng() % (W.dma.size() + 1));
}

void op_waitcnt(uint64_t live, LaneIO* const* io) {
  int vm;
  memcpy(&vm, io[__builtin_ctzll(live)]->in, 4);
  land_dma(g_waves[g_op_wave], (size_t)vm);
}

}  // namespace emu

// ------------------------------------------------------------------ HIP runtime subset

hipError_t hipGetLastError() { return hipSuccess; }
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int) {
  if (attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  *value = emu::g_cus;
  return hipSuccess;
}

// ------------------------------------------------------------------ test controls

namespace {
struct Mapping {
  void* base;
  size_t bytes;
};
std::map<void*, Mapping> g_allocs;
}  // namespace

extern "C" {

// Memory whose end touches an inaccessible page: an access past the last
// 16-byte granule faults.  The pointer is 16-byte aligned.
// A fault inside a kernel is almost always an access past a guarded
// allocation: report the address, the workgroup and work-item, and the
// allocation it is nearest to, then abort.
static void emu_segv(int, siginfo_t* si, void*) {
  char buf[256];
  const uintptr_t a = (uintptr_t)si->si_addr;
  int n = snprintf(buf, sizeof buf, "emulator: memory fault at %p (block %u,%u,%u", si->si_addr,
                   emu::g_bid.x, emu::g_bid.y, emu::g_bid.z);
  if (emu::g_tid) n += snprintf(buf + n, sizeof buf - n, ", thread %u", emu::g_tid->x);
  n += snprintf(buf + n, sizeof buf - n, ")\n");
  if (write(2, buf, n) < 0) {}
  for (auto& kv : g_allocs) {
    const uintptr_t lo = (uintptr_t)kv.second.base, hi = lo + kv.second.bytes;
    if (a >= lo && a < hi) {
      n = snprintf(buf, sizeof buf, "emulator:   inside the mapping of buffer %p (%zu bytes "
                   "mapped): offset %ld from the buffer start\n", kv.first, kv.second.bytes,
                   (long)(a - (uintptr_t)kv.first));
      if (write(2, buf, n) < 0) {}
    }
  }
  signal(SIGSEGV, SIG_DFL);
  abort();
}

static void install_segv_handler() {
  static bool done = false;
  if (done) return;
  done = true;
  struct sigaction sa;
  memset(&sa, 0, sizeof sa);
  sa.sa_sigaction = emu_segv;
  sa.sa_flags = SA_SIGINFO | SA_ONSTACK;
  static char alt[1 << 16];
  stack_t st;
  st.ss_sp = alt;
  st.ss_size = sizeof alt;
  st.ss_flags = 0;
  sigaltstack(&st, nullptr);
  sigaction(SIGSEGV, &sa, nullptr);
}

void* emu_alloc(size_t bytes) {
  install_segv_handler();
  const size_t kPage = 4096;
  const size_t n = (bytes + 15) & ~(size_t)15;
  const size_t pages = (n + kPage - 1) / kPage;
  const size_t total = (pages + 1) * kPage;
  char* m = (char*)mmap(nullptr, total, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS, -1,
                        0);
  if (m == MAP_FAILED) return nullptr;
  mprotect(m + pages * kPage, kPage, PROT_NONE);
  void* p = m + pages * kPage - n;
  g_allocs[p] = Mapping{m, total};
  return p;
}

void emu_free(void* p) {
  auto it = g_allocs.find(p);
  if (it == g_allocs.end()) return;
  munmap(it->second.base, it->second.bytes);
  g_allocs.erase(it);
}

void emu_set_cus(int n) { emu::g_cus = n; }
void emu_set_seed(unsigned long long s) { emu::g_rng.seed(s); }
void emu_counters(unsigned long long* out3) {
  out3[0] = emu::g_blocks;
  out3[1] = emu::g_wave_ops;
  out3[2] = emu::g_barriers;
}

}  // extern "C"
