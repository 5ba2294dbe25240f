// Host runtime of the VerKV C ABI (include/verkv.h): argument checks, workspace
// layout, launches.  No device or host memory is allocated per call; every buffer is
// the caller's.  Compiled by hipcc for gfx950 together with the kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "kernels.h"

using namespace verkv;

namespace {

thread_local char g_last_error[256] = "";

verkv_status hip_fail(hipError_t e, const char *where) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(e));
  return VERKV_EHIP;
}
#define HIP_TRY(expr, where)                          \
  do {                                                \
    hipError_t _e = (expr);                           \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// FNV-1a over the layout of a layer's arrays: with the host cache's address it names the
// rows a workspace's staging area holds.  The sequence lengths are left out: a cache that
// grows (verkv_append) keeps the rows it had, and every staged token is checked against
// the current length.
uint64_t shape_ident(const SeqTable &t, bool bf16) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&](uint64_t v) {
    for (int k = 0; k < 8; ++k) { h ^= (v >> (8 * k)) & 0xFF; h *= 1099511628211ull; }
  };
  mix((uint64_t)t.B); mix((uint64_t)t.Hkv); mix((uint64_t)t.G); mix(bf16 ? 1 : 0);
  for (int b = 0; b < t.B; ++b) mix((uint64_t)t.s[b].cap);
  mix((uint64_t)(uint32_t)t.stage_slots);
  return h;
}

// Build the per-sequence offset table and validate the shape.
verkv_status make_table(const verkv_shape *s, SeqTable &t) {
  if (!s || !s->seq_len) return VERKV_EINVAL;
  if (s->head_dim != VERKV_HEAD_DIM) return VERKV_EUNSUPPORTED;
  if (s->batch < 1 || s->n_kv_heads < 1 || s->group < 1) return VERKV_EINVAL;
  if (s->batch > VERKV_MAX_BATCH || s->group > VERKV_MAX_GROUP) return VERKV_EUNSUPPORTED;
  if (s->n_sink < 0 || s->n_local < 0) return VERKV_EINVAL;
  if (s->kv_dtype != VERKV_BF16 && s->kv_dtype != VERKV_F32) return VERKV_EINVAL;
  std::memset(&t, 0, sizeof(t));
  t.B = s->batch;
  t.Hkv = s->n_kv_heads;
  t.G = s->group;
  t.n_sink = s->n_sink;
  t.n_local = s->n_local;
  int64_t tok = 0, words = 0, chunks = 0;
  for (int b = 0; b < s->batch; ++b) {
    const int32_t n = s->seq_len[b];
    const int32_t cap = s->seq_cap ? s->seq_cap[b] : n;
    if (n < 1 || cap < n) return VERKV_EINVAL;
    if (cap > VERKV_MAX_SEQ_LEN) return VERKV_EUNSUPPORTED;
    t.s[b].n = n;
    t.s[b].cap = cap;
    t.s[b].tok_off = (int32_t)tok;
    t.s[b].word_off = (int32_t)words;
    t.s[b].chunk_off = (int32_t)chunks;
    tok += cap;
    words += words_of(cap);
    chunks += chunks_of(cap);
    t.max_n = std::max(t.max_n, n);
    t.max_cap = std::max(t.max_cap, cap);
  }
  // host-row list entries: the token in the low tok_bits bits, the staging slot + 1 above
  t.tok_bits = 1;
  while ((1 << t.tok_bits) < t.max_cap) ++t.tok_bits;
  t.stage_slots = s->stage_slots;
  if (s->stage_slots < 0 || (int64_t)s->stage_slots > (int64_t)(1ll << (32 - t.tok_bits)) - 1) {
    std::snprintf(g_last_error, sizeof(g_last_error),
                  "stage_slots %d exceeds %lld for a capacity of %d tokens", (int)s->stage_slots,
                  (long long)((1ll << (32 - t.tok_bits)) - 1), (int)t.max_cap);
    return VERKV_EINVAL;
  }
  // longest sequences first: a launch with more workgroups than the device holds at once
  // then starts the longest rows in its first round
  for (int b = 0; b < t.B; ++b) t.order[b] = (uint8_t)b;
  std::stable_sort(t.order, t.order + t.B,
                   [&](uint8_t x, uint8_t y) { return t.s[x].n > t.s[y].n; });
  // every flat index below must stay inside int32 element counts per array
  const int64_t hq = (int64_t)s->n_kv_heads * s->group;
  if (tok * hq > INT32_MAX || chunks * hq * (int64_t)s->n_kv_heads > INT32_MAX) return VERKV_EUNSUPPORTED;
  return VERKV_OK;
}

struct Totals {
  int64_t tok = 0, words = 0, chunks = 0;
};
Totals totals(const SeqTable &t) {
  Totals r;
  for (int b = 0; b < t.B; ++b) {     // array extents: capacities
    r.tok += t.s[b].cap;
    r.words += words_of(t.s[b].cap);
    r.chunks += chunks_of(t.s[b].cap);
  }
  return r;
}

int row_bytes(const verkv_shape *s) { return VERKV_HEAD_DIM * (s->kv_dtype == VERKV_BF16 ? 2 : 4); }

int host_splits(int units) { return std::max(4, std::min(64, 512 / std::max(1, units))); }
// Persistent workers of the pivot attention: PIVOT_WORKERS, or one per schedule chunk
// when there are fewer chunks at most.  Each worker leaves at most one partial per KV
// head it touches, and only its first run can start inside a head, so the partials of a
// step number at most workers + KV heads.
int pivot_workers(int cap, int units) {
  const int64_t chunks = (int64_t)units * ((cap + PIVOT_CHUNK - 1) / PIVOT_CHUNK);
  return (int)std::max<int64_t>(1, std::min<int64_t>(PIVOT_WORKERS, chunks));
}
int pivot_slots(int cap, int units) { return pivot_workers(cap, units) + units; }
// Rows of piv_k / piv_v: the schedule stores worker w's i-th chunk as block i P + w, and
// the workers' chunk counts differ by at most one, so ceil(NC / P) P <= NC + P - 1 blocks.
int64_t pivot_rows(int cap, int units) {
  const int64_t nc_max = (int64_t)units * ((cap + PIVOT_CHUNK - 1) / PIVOT_CHUNK);
  return (nc_max + PIVOT_WORKERS) * PIVOT_CHUNK;
}

// Workgroups per query row in the decision kernel, as sized in the workspace: enough
// to give 256 CUs two workgroups each, at least TEAM_MIN_TOKENS tokens per workgroup,
// at most TEAM_MAX.  At launch it is lowered further if fewer can be co-resident.
int team_size(int rows, int max_n) {
  const int by_cu = 512 / std::max(1, rows);
  const int by_len = (max_n + TEAM_MIN_TOKENS - 1) / TEAM_MIN_TOKENS;
  return std::max(1, std::min(TEAM_MAX, std::min(by_cu, by_len)));
}

// Host rows staged per KV head: the shape's stage_slots, or by default up to
// STAGE_SLOTS_DEFAULT per KV head and STAGE_ROWS_TOTAL in all, within what a list entry
// can name.
int stage_rows_of(const SeqTable &t, int units) {
  if (t.stage_slots > 0) return t.stage_slots;
  const int64_t lim = (1ll << (32 - t.tok_bits)) - 1;
  return (int)std::min<int64_t>(lim, std::min(STAGE_SLOTS_DEFAULT, STAGE_ROWS_TOTAL / std::max(1, units)));
}

// Decode workspace layout.
struct DecodeWs {
  size_t wc, cstat, cscale, fbits, h2d, coef, ppart, hpart, status;
  size_t xseq, wcount, part, hcnt, hbeta, hV, hmax, wkey, wlo, apart, cf0, bprev;
  size_t stage, stage_tok, slot_of, pf_new, pf_slot, pf_cnt, shdr, h2dc, stg, psched, pruns, gpar;
  int srows;
  size_t total;
  int nsp, nsh, team;      // nsp: pivot partial slots
};
DecodeWs decode_layout(const SeqTable &t, int cap, bool bf16, bool staging = true) {
  const Totals T = totals(t);
  const int64_t Hq = (int64_t)t.Hkv * t.G;
  const int units = t.B * t.Hkv;
  const int64_t rows = (int64_t)units * t.G;
  DecodeWs w;
  w.nsp = pivot_slots(cap, units);
  w.nsh = host_splits(units);
  w.team = team_size((int)rows, t.max_cap);      // sized for the longest the arrays may hold
  const int64_t tm = w.team > 1 ? w.team : 0;       // member histograms only for teams
  size_t off = 0;
  w.xseq = off;   off = align_up(off + 8 * (size_t)(rows * 2 * w.team));
  w.wcount = off; off = align_up(off + 4 * (size_t)rows);
  w.part = off;   off = align_up(off + 8 * (size_t)(rows * 2 * w.team * PART));
  w.apart = off;  off = align_up(off + 8 * (size_t)(rows * w.team * 8));
  w.hcnt = off;   off = align_up(off + 4 * (size_t)(rows * 2 * tm * NBUCKET));   // two buffers
  w.hbeta = off;  off = align_up(off + 8 * (size_t)(rows * 2 * tm * NBUCKET));
  w.hV = off;     off = align_up(off + 8 * (size_t)(rows * 2 * tm * NBUCKET));
  w.hmax = off;   off = align_up(off + 8 * (size_t)(rows * 2 * tm * NBUCKET));
  const int64_t mm = w.team > 1 ? 1 : 0;
  w.wkey = off;   off = align_up(off + 8 * (size_t)(rows * mm * WIN));
  w.wlo = off;    off = align_up(off + 4 * (size_t)(rows * mm * WIN));
  w.wc = off;     off = align_up(off + 8 * (size_t)(Hq * T.tok));
  w.cstat = off;  off = align_up(off + 16 * (size_t)(Hq * T.chunks));
  w.cf0 = off;    off = align_up(off + 8 * (size_t)(Hq * T.chunks));
  w.cscale = off; off = align_up(off + 8 * (size_t)(Hq * T.chunks));
  w.fbits = off;  off = align_up(off + 4 * (size_t)(t.Hkv * T.words));
  w.h2d = off;    off = align_up(off + 4 * (size_t)(t.Hkv * T.tok));
  w.coef = off;   off = align_up(off + 4 * (size_t)(t.B * Hq * (int64_t)cap));
  w.ppart = off;  off = align_up(off + 4 * (size_t)w.nsp * t.G * (D + 1));
  w.hpart = off;  off = align_up(off + 4 * (size_t)units * w.nsh * t.G * (D + 1));
  w.status = off; off = align_up(off + 64);
  w.bprev = off;  off = align_up(off + 8 * (size_t)rows);
  // cross-step staging of host rows: srows rows of the cache's dtype per KV head, the
  // maps between slots and tokens, and the plan of each step
  w.srows = !staging ? 0 : stage_rows_of(t, units);
  w.stage = off;     off = align_up(off + (size_t)units * w.srows * D * (bf16 ? 2 : 4));
  w.stage_tok = off; off = align_up(off + 4 * (size_t)units * w.srows);
  w.slot_of = off;   off = align_up(off + (w.srows > 0 ? 4 * (size_t)(t.Hkv * T.tok) : 0));
  w.pf_new = off;    off = align_up(off + 4 * (size_t)units * w.srows);
  w.pf_slot = off;   off = align_up(off + 4 * (size_t)units * w.srows);
  w.pf_cnt = off;    off = align_up(off + 4 * (size_t)units);
  w.shdr = off;      off = align_up(off + 8 * (size_t)STAGE_HDR_WORDS);
  w.h2dc = off;      off = align_up(off + 4 * (size_t)units);
  w.stg = off;       off = align_up(off + 4 * (size_t)units);   // staged rows the host-row kernel used
  w.psched = off;    off = align_up(off + 16 * (size_t)(2 * PIVOT_WORKERS + 1));
  w.pruns = off;     off = align_up(off + 16 * (size_t)units);
  w.gpar = off;      off = align_up(off + 32 * (size_t)rows);
  w.total = off;
  return w;
}

struct CompressWs {
  size_t ka, kb, status, psched, pruns, total;
};
CompressWs compress_layout(const SeqTable &t) {
  const Totals T = totals(t);
  CompressWs w;
  size_t off = 0;
  w.ka = off;     off = align_up(off + 8 * (size_t)(t.Hkv * T.tok));
  w.kb = off;     off = align_up(off + 8 * (size_t)(t.Hkv * T.tok));
  w.status = off; off = align_up(off + 64);
  w.psched = off; off = align_up(off + 16 * (size_t)(2 * PIVOT_WORKERS + 1));
  w.pruns = off;  off = align_up(off + 16 * (size_t)(t.B * t.Hkv));
  w.total = off;
  return w;
}

// A host-cache pointer as the kernels must see it: pinned host memory is translated
// to its device-visible address; device memory is used as is.
verkv_status device_view(const void *p, const void **out) {
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    std::snprintf(g_last_error, sizeof(g_last_error), "host cache pointer is not pinned or device memory");
    return VERKV_EINVAL;
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
    *out = p;
    return VERKV_OK;
  }
  if (attr.type == hipMemoryTypeHost) {
    void *d = nullptr;
    e = hipHostGetDevicePointer(&d, const_cast<void *>(p), 0);
    if (e != hipSuccess || !d) {
      (void)hipGetLastError();
      std::snprintf(g_last_error, sizeof(g_last_error), "pinned host cache is not mapped for the device");
      return VERKV_EINVAL;
    }
    *out = d;
    return VERKV_OK;
  }
  std::snprintf(g_last_error, sizeof(g_last_error), "host cache pointer is pageable memory");
  return VERKV_EINVAL;
}

// Co-resident decision workgroups on the current device for a team size (the LDS the
// kernel reserves depends on the slice each member holds).
int decide_capacity(int max_n, int team) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  return cus * decide_blocks_per_cu(max_n, team);
}

// ---------------------------------------------------------------- side stream
// verkv_refine runs the resident-pivot attention and the eps_after pass on a second
// stream of the library (default priority) while the host-row kernel, bound by the host
// link, runs on the caller's stream; both are joined before the finishing kernel.  One
// stream and one event pair per device, created on first use; the fork and join of one
// call are recorded under a per-device lock.
struct Side {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, pref = nullptr, dec = nullptr;
  std::mutex mu;
};
constexpr int MAX_DEVICES = 64;
Side g_side[MAX_DEVICES];
std::mutex g_side_init;

verkv_status side_for_device(Side **out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return VERKV_EUNSUPPORTED;
  Side &sd = g_side[dev];
  std::lock_guard<std::mutex> lk(g_side_init);
  if (!sd.s) {
    HIP_TRY(hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking), "hipStreamCreateWithFlags");
    HIP_TRY(hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming), "hipEventCreateWithFlags");
    HIP_TRY(hipEventCreateWithFlags(&sd.join, hipEventDisableTiming), "hipEventCreateWithFlags");
    HIP_TRY(hipEventCreateWithFlags(&sd.pref, hipEventDisableTiming), "hipEventCreateWithFlags");
    HIP_TRY(hipEventCreateWithFlags(&sd.dec, hipEventDisableTiming), "hipEventCreateWithFlags");
  }
  *out = &sd;
  return VERKV_OK;
}

// ---------------------------------------------------------------- optional kernel timing
enum KernelId { K_POISSON = 0, K_GATHER, K_SKETCH, K_DECIDE, K_UNION, K_PIVOT, K_HOST, K_FINISH, K_AFTER,
                K_COEF, K_PREFETCH, K_QUANT, K_RESOLVE, K_PLAN, K_COUNT };
struct Profiler {
  bool on = false;
  std::vector<hipEvent_t> ev;       // pairs
  std::vector<int> kind;
  size_t used = 0;
};
Profiler g_prof;
}  // namespace
namespace verkv {
thread_local LaunchEvents g_launch_ev;
}
namespace {

// Hands the next launch an event pair; the launcher has the dispatch stamp them.
struct Timed {
  int slot = -1;
  Timed(int kid, hipStream_t) {
    if (g_prof.on && g_prof.used < g_prof.kind.size()) {
      slot = (int)g_prof.used++;
      g_prof.kind[slot] = kid;
      g_launch_ev = {g_prof.ev[2 * slot], g_prof.ev[2 * slot + 1], false};
    }
  }
  ~Timed() {
    if (slot >= 0 && !g_launch_ev.used) g_prof.kind[slot] = -1;   // the launch failed early
    g_launch_ev = LaunchEvents{};
  }
};

// ---------------------------------------------------------------- static scratch
// The workspace of verkv_step_noalloc: a file-scope device array (each device the
// library runs on holds its own copy until the process ends).  In host code `scratch`
// names a host-side stand-in, not device memory; its device address is looked up once
// per device with hipGetSymbolAddress and only that address is handed to the kernels.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[STATIC_SCRATCH_BYTES];

struct ScratchPtr {
  void *p = nullptr;
  bool set = false;
};
ScratchPtr g_scratch[MAX_DEVICES];
std::mutex g_scratch_mu;

verkv_status scratch_for_device(uint8_t **out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return VERKV_EUNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  ScratchPtr &sp = g_scratch[dev];
  if (!sp.set) {
    void *ptr = nullptr;
    HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress");
    if (!ptr) {
      std::snprintf(g_last_error, sizeof(g_last_error), "static scratch has no device address");
      return VERKV_EHIP;
    }
    sp.p = ptr;
    sp.set = true;
  }
  *out = static_cast<uint8_t *>(sp.p);
  return VERKV_OK;
}

}  // namespace

extern "C" {

int32_t verkv_version(void) { return 109; }

#ifndef VERKV_SOURCE_HASH
#define VERKV_SOURCE_HASH "unknown"
#endif
const char *verkv_source_hash(void) { return VERKV_SOURCE_HASH; }

const char *verkv_status_str(int32_t s) {
  switch (s) {
    case VERKV_OK: return "ok";
    case VERKV_EINVAL: return "invalid argument";
    case VERKV_EBUDGET: return "budget below the forced sink + local tokens";
    case VERKV_ECAPACITY: return "pivot capacity exceeded";
    case VERKV_EHIP: return "HIP runtime error";
    case VERKV_EUNSUPPORTED: return "unsupported shape";
    case VERKV_EWORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char *verkv_last_error(void) { return g_last_error; }

}  // extern "C"

namespace {
struct AppendWs {
  size_t plan, plan_r, sold, rold, snew, rnew, rows_k, rows_v, total;
};
AppendWs append_layout(const SeqTable &t, int cap, int row_bytes) {
  const int64_t units = (int64_t)t.B * t.Hkv;
  AppendWs w;
  size_t off = 0;
  w.plan = off;   off = align_up(off + 16 * (size_t)units);
  w.plan_r = off; off = align_up(off + 8 * (size_t)units);
  w.sold = off;   off = align_up(off + 16 * (size_t)(2 * PIVOT_WORKERS + 1));
  w.rold = off;   off = align_up(off + 16 * (size_t)units);
  w.snew = off;   off = align_up(off + 16 * (size_t)(2 * PIVOT_WORKERS + 1));
  w.rnew = off;   off = align_up(off + 16 * (size_t)units);
  w.rows_k = off; off = align_up(off + (size_t)units * cap * row_bytes);
  w.rows_v = off; off = align_up(off + (size_t)units * cap * row_bytes);
  w.total = off;
  return w;
}
}  // namespace

extern "C" {

size_t verkv_append_workspace_bytes(const verkv_shape *s, int32_t cap) {
  SeqTable t;
  if (cap < 1 || make_table(s, t) != VERKV_OK) return 0;
  return append_layout(t, cap, row_bytes(s)).total;
}

verkv_status verkv_append(const verkv_shape *s, verkv_state *st, const float *tau,
                          const void *K_host, const void *V_host, uint64_t seed, int32_t *status,
                          void *workspace, size_t workspace_bytes, verkv_stream_t stream_) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  SeqTable t;
  verkv_status rc = make_table(s, t);
  if (rc != VERKV_OK) return rc;
  if (!st || !tau || !K_host || !V_host || !status || !workspace) return VERKV_EINVAL;
  if (!st->r || !st->resident || !st->piv_idx || !st->piv_count || !st->piv_k || !st->piv_v ||
      !st->level || st->cap < 1)
    return VERKV_EINVAL;
  for (int b = 0; b < t.B; ++b) {
    if (t.s[b].n + 1 > t.s[b].cap) {
      std::snprintf(g_last_error, sizeof(g_last_error),
                    "sequence %d has no capacity left (length %d, capacity %d)", b, t.s[b].n,
                    t.s[b].cap);
      return VERKV_EINVAL;
    }
  }
  const int rb = row_bytes(s);
  const AppendWs L = append_layout(t, st->cap, rb);
  if (workspace_bytes < L.total) return VERKV_EWORKSPACE;
  const void *Kd = nullptr, *Vd = nullptr;
  if ((rc = device_view(K_host, &Kd)) != VERKV_OK) return rc;
  if ((rc = device_view(V_host, &Vd)) != VERKV_OK) return rc;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  const int units = t.B * t.Hkv;
  AppendArgs a;
  a.t = t;
  a.tau = tau;
  a.level = st->level;
  a.r = st->r;
  a.resident = st->resident;
  a.piv_idx = st->piv_idx;
  a.piv_count = st->piv_count;
  a.cap = st->cap;
  a.seed = seed;
  a.layer = s->layer;
  a.status = status;
  a.plan = reinterpret_cast<int4 *>(ws + L.plan);
  a.plan_r = reinterpret_cast<double *>(ws + L.plan_r);
  a.K_host = static_cast<const uint8_t *>(Kd);
  a.V_host = static_cast<const uint8_t *>(Vd);
  a.piv_k = static_cast<uint8_t *>(st->piv_k);
  a.piv_v = static_cast<uint8_t *>(st->piv_v);
  a.rows_k = ws + L.rows_k;
  a.rows_v = ws + L.rows_v;
  a.sched_old = reinterpret_cast<const int4 *>(ws + L.sold);
  a.runs_old = reinterpret_cast<const int4 *>(ws + L.rold);
  a.sched_new = reinterpret_cast<const int4 *>(ws + L.snew);
  a.runs_new = reinterpret_cast<const int4 *>(ws + L.rnew);
  a.workers = pivot_workers(st->cap, units);
  a.row_bytes = rb;
  a.rows = pivot_rows(st->cap, units);
  // the schedule of the counts before and after the append, for the pivot rows' places
  PlanArgs pl;
  pl.t = t;
  pl.piv_count = st->piv_count;
  pl.cap = st->cap;
  pl.workers = a.workers;
  pl.sched = reinterpret_cast<int4 *>(ws + L.sold);
  pl.runs = reinterpret_cast<int4 *>(ws + L.rold);
  HIP_TRY(launch_append_plan(a, units, stream), "append plan launch");
  HIP_TRY(launch_pivot_schedule(pl, stream), "pivot schedule launch");
  HIP_TRY(launch_append_copy(a, units, false, stream), "append copy-out launch");
  HIP_TRY(launch_append_apply(a, units, stream), "append apply launch");
  pl.sched = reinterpret_cast<int4 *>(ws + L.snew);
  pl.runs = reinterpret_cast<int4 *>(ws + L.rnew);
  HIP_TRY(launch_pivot_schedule(pl, stream), "pivot schedule launch");
  HIP_TRY(launch_append_copy(a, units, true, stream), "append copy-in launch");
  return VERKV_OK;
}

size_t verkv_compress_workspace_bytes(const verkv_shape *s) {
  SeqTable t;
  if (make_table(s, t) != VERKV_OK) return 0;
  return compress_layout(t).total;
}

verkv_status verkv_quantize_sketch(const verkv_shape *s, const void *K, void *sketch,
                                   verkv_stream_t stream_) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  SeqTable t;
  verkv_status rc = make_table(s, t);
  if (rc != VERKV_OK) return rc;
  if (!K || !sketch) return VERKV_EINVAL;
  const void *Kd = nullptr;
  if ((rc = device_view(K, &Kd)) != VERKV_OK) return rc;
  QuantArgs qa;
  qa.K = static_cast<const uint8_t *>(Kd);
  qa.out = static_cast<uint8_t *>(sketch);
  qa.rows = (int64_t)t.Hkv * totals(t).tok;
  {
    Timed tm(K_QUANT, stream);
    HIP_TRY(launch_quant_sketch(qa, s->kv_dtype == VERKV_BF16, stream), "quantise launch");
  }
  return VERKV_OK;
}

size_t verkv_pivot_rows(const verkv_shape *s, int32_t cap) {
  SeqTable t;
  if (make_table(s, t) != VERKV_OK || cap < 1) return 0;
  return (size_t)pivot_rows(cap, t.B * t.Hkv);
}

size_t verkv_decode_workspace_bytes(const verkv_shape *s, int32_t cap) {
  SeqTable t;
  if (cap < 1 || make_table(s, t) != VERKV_OK) return 0;
  return decode_layout(t, cap, s->kv_dtype == VERKV_BF16).total;
}

verkv_status verkv_staged_rows(void *workspace, size_t workspace_bytes, const verkv_shape *s,
                               int32_t cap, verkv_stream_t stream_, int64_t *rows) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  SeqTable t;
  verkv_status rc = make_table(s, t);
  if (rc != VERKV_OK) return rc;
  if (!workspace || !rows || cap < 1) return VERKV_EINVAL;
  const DecodeWs L = decode_layout(t, cap, s->kv_dtype == VERKV_BF16);
  if (workspace_bytes < L.total) return VERKV_EWORKSPACE;
  const int units = t.B * t.Hkv;
  std::vector<int32_t> cnt((size_t)units, 0);
  HIP_TRY(hipMemcpyAsync(cnt.data(), static_cast<uint8_t *>(workspace) + L.stg,
                         sizeof(int32_t) * (size_t)units, hipMemcpyDeviceToHost, stream),
          "hipMemcpyAsync");
  HIP_TRY(hipStreamSynchronize(stream), "hipStreamSynchronize");
  int64_t sum = 0;
  for (int32_t c : cnt) sum += c;
  *rows = sum;
  return VERKV_OK;
}

verkv_status verkv_compress(const verkv_shape *s, const float *tau, const void *K_host,
                            const void *V_host, double eta, uint64_t seed, verkv_state *st,
                            void *workspace, size_t workspace_bytes, int32_t *needed_cap,
                            verkv_stream_t stream_) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  SeqTable t;
  verkv_status rc = make_table(s, t);
  if (rc != VERKV_OK) return rc;
  if (!tau || !K_host || !V_host || !st || !workspace) return VERKV_EINVAL;
  if (!st->r || !st->resident || !st->piv_idx || !st->piv_count || !st->piv_k || !st->piv_v ||
      st->cap < 1)
    return VERKV_EINVAL;
  if (!(eta > 0.0 && eta <= 1.0)) return VERKV_EINVAL;
  for (int b = 0; b < t.B; ++b) {
    const int n = t.s[b].n;
    const int forced = std::min(n, s->n_sink + s->n_local);
    if (eta * (double)n - (double)forced < 0.0) return VERKV_EBUDGET;
  }
  const CompressWs L = compress_layout(t);
  if (workspace_bytes < L.total) return VERKV_EWORKSPACE;
  const void *Kd = nullptr, *Vd = nullptr;
  if ((rc = device_view(K_host, &Kd)) != VERKV_OK) return rc;
  if ((rc = device_view(V_host, &Vd)) != VERKV_OK) return rc;

  uint8_t *ws = static_cast<uint8_t *>(workspace);
  int32_t *status = reinterpret_cast<int32_t *>(ws + L.status);
  HIP_TRY(hipMemsetAsync(status, 0, 16, stream), "hipMemsetAsync");
  CompressArgs a;
  a.t = t;
  a.tau = tau;
  a.eta = eta;
  a.seed = seed;
  a.layer = s->layer;
  a.r = st->r;
  a.resident = st->resident;
  a.piv_idx = st->piv_idx;
  a.piv_count = st->piv_count;
  a.cap = st->cap;
  a.keys_a = reinterpret_cast<uint64_t *>(ws + L.ka);
  a.keys_b = reinterpret_cast<uint64_t *>(ws + L.kb);
  a.status = status;
  a.level = st->level;
  const int units = t.B * t.Hkv;
  {
    Timed tm(K_POISSON, stream);
    HIP_TRY(launch_poissoncomp(a, units, stream), "poissoncomp launch");
  }
  int32_t hstat[2] = {0, 0};
  HIP_TRY(hipMemcpyAsync(hstat, status, sizeof(hstat), hipMemcpyDeviceToHost, stream), "hipMemcpyAsync");
  HIP_TRY(hipStreamSynchronize(stream), "hipStreamSynchronize");
  if (hstat[0] & 1) {
    std::snprintf(g_last_error, sizeof(g_last_error), "tau outside [0, 1]");
    return VERKV_EINVAL;
  }
  if (hstat[1] > st->cap) {
    if (needed_cap) *needed_cap = hstat[1];
    return VERKV_ECAPACITY;
  }
  if (needed_cap) *needed_cap = hstat[1];
  // the pivot-attention schedule of these pivot counts: the gather stores the rows in
  // the order the attention kernel's workers read them
  PlanArgs pl;
  pl.t = t;
  pl.piv_count = st->piv_count;
  pl.cap = st->cap;
  pl.workers = pivot_workers(st->cap, units);
  pl.sched = reinterpret_cast<int4 *>(ws + L.psched);
  pl.runs = reinterpret_cast<int4 *>(ws + L.pruns);
  HIP_TRY(launch_pivot_schedule(pl, stream), "pivot schedule launch");
  GatherArgs gth;
  gth.t = t;
  gth.K_host = static_cast<const uint8_t *>(Kd);
  gth.V_host = static_cast<const uint8_t *>(Vd);
  gth.piv_idx = st->piv_idx;
  gth.piv_count = st->piv_count;
  gth.piv_k = static_cast<uint8_t *>(st->piv_k);
  gth.piv_v = static_cast<uint8_t *>(st->piv_v);
  gth.cap = st->cap;
  gth.row_bytes = row_bytes(s);
  gth.sched = pl.sched;
  gth.runs = pl.runs;
  gth.workers = pl.workers;
  gth.rows = pivot_rows(st->cap, units);
  {
    Timed tm(K_GATHER, stream);
    HIP_TRY(launch_gather_pivots(gth, units, stream), "gather launch");
  }
  return VERKV_OK;
}

static verkv_status check_step(const verkv_shape *s, const verkv_state *st, const float *q,
                               const verkv_step_out *out, SeqTable &t) {
  verkv_status rc = make_table(s, t);
  if (rc != VERKV_OK) return rc;
  if (!st || !q || !out) return VERKV_EINVAL;
  if (!st->r || !st->resident || !st->piv_idx || !st->piv_count || !st->piv_k || !st->piv_v ||
      !st->sketch || st->cap < 1)
    return VERKV_EINVAL;
  if (st->sketch_format != VERKV_SKETCH_ROWS && st->sketch_format != VERKV_SKETCH_2BIT) return VERKV_EINVAL;
  if (st->sketch_format == VERKV_SKETCH_2BIT && st->sketch_exact) {
    std::snprintf(g_last_error, sizeof(g_last_error), "a 2-bit sketch is not exact (sketch_exact must be 0)");
    return VERKV_EINVAL;
  }
  return VERKV_OK;
}

// The caches the step's prefetch reads, resolved to their device views before anything
// is enqueued: the value cache (v_host), and with a sketch that is not exact the key
// cache too (k_host; without it that mode stages nothing).  *Vd stays null when there
// is no prefetch; *Kd is set only when keys are staged.
static verkv_status prefetch_source(const verkv_state *st, int srows, const void **Vd,
                                    const void **Kd) {
  *Vd = nullptr;
  *Kd = nullptr;
  if (!st->v_host || srows <= 0) return VERKV_OK;
  if (!st->sketch_exact && !st->k_host) return VERKV_OK;
  verkv_status rc = device_view(st->v_host, Vd);
  if (rc == VERKV_OK && !st->sketch_exact) rc = device_view(st->k_host, Kd);
  if (rc != VERKV_OK) *Vd = nullptr;
  return rc;
}

// Staging slots: the workspace reserves srows rows of the cache's dtype per KV head; a
// slot holds the value row, or the value and the key row (keys staged), so with keys
// the slot count halves.
struct StageGeom {
  int rows;
  int stride;
  bool kv;
};
static StageGeom stage_geom(int srows, bool bf16, bool kv) {
  const int row = VERKV_HEAD_DIM * (bf16 ? 2 : 4);
  return StageGeom{kv ? srows / 2 : srows, kv ? 2 * row : row, kv};
}

// The identity staged rows are published under: the shape, and the key cache's
// address when keys are staged beside the values (the value cache's address is the
// other half).
static uint64_t stage_ident(const SeqTable &t, bool bf16, const void *Kd) {
  uint64_t h = shape_ident(t, bf16);
  const uint64_t k = reinterpret_cast<uint64_t>(Kd);
  for (int i = 0; i < 8; ++i) { h ^= (k >> (8 * i)) & 0xFF; h *= 1099511628211ull; }
  return h;
}

// The pivot-coefficient pass of a step on workspace ws (with the pivot attention's
// schedule in its extra workgroup).
static UnionArgs coef_args(const SeqTable &t, const verkv_state *st, uint8_t *ws, const DecodeWs &L,
                           const verkv_step_out *out, int units) {
  UnionArgs un;
  un.t = t;
  un.fbits = reinterpret_cast<const uint32_t *>(ws + L.fbits);
  un.resident = st->resident;
  un.piv_idx = st->piv_idx;
  un.piv_count = st->piv_count;
  un.cap = st->cap;
  un.r = st->r;
  un.wc = reinterpret_cast<const double *>(ws + L.wc);
  un.cscale = reinterpret_cast<const double *>(ws + L.cscale);
  un.beta_star = out->beta_star;
  un.kappa = 0.0;
  un.params = reinterpret_cast<const double *>(ws + L.status + 32);   // kappa of the step
  un.fetch_idx = nullptr;
  un.fetch_cap = 0;
  un.fetch_count = nullptr;
  un.h2d_count = nullptr;
  un.h2d_idx = nullptr;
  un.coef = reinterpret_cast<float *>(ws + L.coef);
  un.coef_pass = 1;
  un.slot_of = nullptr;
  un.stage_rows = 0;
  un.shdr = nullptr;
  un.ident_ptr = 0;
  un.ident_shape = 0;
  un.h2d_count_ws = nullptr;
  un.stg_cnt = nullptr;
  un.piv_sched = reinterpret_cast<int4 *>(ws + L.psched);
  un.piv_runs = reinterpret_cast<int4 *>(ws + L.pruns);
  un.piv_workers = pivot_workers(st->cap, units);
  return un;
}

// The partial certificate terms of eps_after = eps_hat(L \ F): they need only the
// decisions of the step.
static verkv_status launch_after_terms(const SeqTable &t, const verkv_state *st,
                                       const verkv_step_out *out, uint8_t *ws, const DecodeWs &L,
                                       hipStream_t s) {
  AfterArgs af;
  af.t = t;
  af.wc = reinterpret_cast<const double *>(ws + L.wc);
  af.cscale = reinterpret_cast<const double *>(ws + L.cscale);
  af.r = st->r;
  af.fbits = reinterpret_cast<const uint32_t *>(ws + L.fbits);
  af.beta_star = out->beta_star;
  af.params = reinterpret_cast<const double *>(ws + L.status + 32);
  af.team = L.team;
  af.part = reinterpret_cast<double *>(ws + L.apart);
  Timed tm(K_AFTER, s);
  HIP_TRY(launch_after(af, t.B * t.Hkv * t.G, s), "eps_after launch");
  return VERKV_OK;
}

// The staging arguments of a step on workspace ws: the copies (decode) and the plan for
// the next step (refine) share them.
static PrefetchArgs stage_args(const SeqTable &t, uint8_t *ws, const DecodeWs &L, const void *Vd,
                               const void *Kd, bool bf16, const StageGeom &sg) {
  PrefetchArgs pa;
  pa.t = t;
  pa.prev_list = reinterpret_cast<const int32_t *>(ws + L.h2d);
  pa.prev_count = reinterpret_cast<const int32_t *>(ws + L.h2dc);
  pa.vrows = static_cast<const uint8_t *>(Vd);
  pa.krows = static_cast<const uint8_t *>(Kd);
  pa.stage = ws + L.stage;
  pa.stage_tok = reinterpret_cast<int32_t *>(ws + L.stage_tok);
  pa.slot_of = reinterpret_cast<int32_t *>(ws + L.slot_of);
  pa.pf_new = reinterpret_cast<int32_t *>(ws + L.pf_new);
  pa.pf_slot = reinterpret_cast<int32_t *>(ws + L.pf_slot);
  pa.pf_count = reinterpret_cast<int32_t *>(ws + L.pf_cnt);
  pa.shdr = reinterpret_cast<uint64_t *>(ws + L.shdr);
  pa.ident_ptr = reinterpret_cast<uint64_t>(Vd);
  pa.ident_shape = stage_ident(t, bf16, Kd);
  pa.stage_rows = sg.rows;
  pa.stage_stride = sg.stride;
  return pa;
}

// How a step uses the library's resources: the ordinary entry points stage host rows
// across steps and run the refine side of a step on the library's second stream; the
// allocation-free entry point does neither (everything on the caller's stream) and may
// take the kernels' status flags in a caller-owned word instead of the workspace's.
struct StepMode {
  bool staging = true;
  bool side = true;
  int32_t *status = nullptr;
  uint32_t flags = 0;        // VERKV_STEP_* of verkv_decode_step_ex
};

// Argument checks of KVFetch steps 1-4 (nothing is enqueued).
static verkv_status decode_args(const verkv_shape *s, const verkv_state *st, const float *q,
                                double beta, double eps, double delta, const verkv_step_out *out,
                                SeqTable &t) {
  verkv_status rc = check_step(s, st, q, out, t);
  if (rc != VERKV_OK) return rc;
  if (!(beta >= 0.0) || !(eps > 0.0) || !(delta > 0.0 && delta < 1.0)) return VERKV_EINVAL;
  if (!out->m_hat || !out->d_sketch || !out->beta_star || !out->eps_hat || !out->certified ||
      !out->kstar || !out->fetch_count || !out->h2d_count)
    return VERKV_EINVAL;
  if (out->fetch_idx && out->fetch_cap < 1) return VERKV_EINVAL;
  return VERKV_OK;
}

// Argument checks of KVFetch step 5; resolves the host caches to their device views.
static verkv_status refine_args(const verkv_shape *s, const verkv_state *st, const float *q,
                                const void *K_host, const void *V_host, const verkv_step_out *out,
                                SeqTable &t, const void **Kd, const void **Vd) {
  verkv_status rc = check_step(s, st, q, out, t);
  if (rc != VERKV_OK) return rc;
  if (!K_host || !V_host || !out->eps_after || !out->n_hat || !out->d_hat || !out->o ||
      !out->lse || !out->m_hat || !out->d_sketch || !out->beta_star || !out->h2d_count)
    return VERKV_EINVAL;
  if ((rc = device_view(K_host, Kd)) != VERKV_OK) return rc;
  return device_view(V_host, Vd);
}

static verkv_status decode_impl(const verkv_shape *s, const verkv_state *st, const float *q,
                                double beta, double eps, double delta, verkv_step_out *out,
                                void *workspace, size_t workspace_bytes, hipStream_t stream,
                                const StepMode &mode) {
  SeqTable t;
  verkv_status rc = decode_args(s, st, q, beta, eps, delta, out, t);
  if (rc != VERKV_OK) return rc;
  if (!workspace) return VERKV_EINVAL;
  const bool bf16 = s->kv_dtype == VERKV_BF16;
  const DecodeWs L = decode_layout(t, st->cap, bf16, mode.staging);
  if (workspace_bytes < L.total) return VERKV_EWORKSPACE;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  const Totals T = totals(t);
  const int units = t.B * t.Hkv;
  const int rows = units * t.G;
  // every argument and the library's second stream are resolved before the first launch
  const void *Vd = nullptr, *Kd = nullptr;
  if (mode.side && (rc = prefetch_source(st, L.srows, &Vd, &Kd)) != VERKV_OK) return rc;
  const bool prefetch = Vd != nullptr;   // host cache(s) and staging rows
  const StageGeom sg = stage_geom(L.srows, bf16, Kd != nullptr);
  Side *sd = nullptr;
  if (mode.side && (rc = side_for_device(&sd)) != VERKV_OK) return rc;

  SketchArgs sk;
  sk.t = t;
  sk.sketch = static_cast<const uint8_t *>(st->sketch);
  sk.q2 = st->sketch_format == VERKV_SKETCH_2BIT ? 1 : 0;
  sk.q = q;
  sk.inv_sqrt_d = 1.0 / std::sqrt((double)VERKV_HEAD_DIM);
  sk.wc = reinterpret_cast<double *>(ws + L.wc);
  sk.cstat = reinterpret_cast<double2 *>(ws + L.cstat);
  sk.r = st->r;
  sk.cf0 = reinterpret_cast<double *>(ws + L.cf0);
  sk.fbits = reinterpret_cast<uint32_t *>(ws + L.fbits);
  sk.wcount = reinterpret_cast<uint32_t *>(ws + L.wcount);
  sk.xseq = reinterpret_cast<double *>(ws + L.xseq);
  sk.xseq_row = 2 * L.team;
  sk.kstar = out->kstar;
  sk.total_blocks = (int32_t)(t.Hkv * T.chunks);
  {
    Timed tm(K_SKETCH, stream);
    HIP_TRY(launch_sketch(sk, bf16, stream), "sketch launch");
  }

  // staging copies on the library's second stream, beside the decision kernel (they
  // start after the sketch kernel, which needs every register of the CUs): the rows the
  // plan of the previous step on this workspace brings in.  The fork point is the end of
  // the sketch kernel; the copies are enqueued after the decision kernel, so that the
  // decision workgroups are placed on the CUs before the copy blocks are (enqueued
  // first, they delayed the start of the last team members by 13-15 us).
  std::unique_lock<std::mutex> lk;
  if (mode.side) lk = std::unique_lock<std::mutex>(sd->mu);
  PrefetchArgs pa;
  if (prefetch) {
    HIP_TRY(hipEventRecord(sd->fork, stream), "hipEventRecord");
    pa = stage_args(t, ws, L, Vd, Kd, bf16, sg);
  }
  auto launch_pf = [&]() -> verkv_status {
    if (!prefetch) return VERKV_OK;
    HIP_TRY(hipStreamWaitEvent(sd->s, sd->fork, 0), "hipStreamWaitEvent");
    {
      Timed tm(K_PREFETCH, sd->s);
      HIP_TRY(launch_stage_fetch(pa, units, bf16, sd->s), "staging copy launch");
    }
    HIP_TRY(hipEventRecord(sd->pref, sd->s), "hipEventRecord");
    return VERKV_OK;
  };

  DecideArgs dc;
  dc.t = t;
  dc.wc = sk.wc;
  dc.cstat = sk.cstat;
  dc.cf0 = sk.cf0;
  dc.cscale = reinterpret_cast<double *>(ws + L.cscale);
  dc.r = st->r;
  dc.fbits = sk.fbits;
  dc.kappa = beta;
  dc.eps = eps;
  dc.l = std::log(2.0 / delta);
  dc.m_hat = out->m_hat;
  dc.d_sketch = out->d_sketch;
  dc.beta_star = out->beta_star;
  dc.eps_hat = out->eps_hat;
  dc.certified = out->certified;
  dc.kstar = out->kstar;
  dc.status = mode.status ? mode.status : reinterpret_cast<int32_t *>(ws + L.status);
  dc.params = reinterpret_cast<double *>(ws + L.status + 32);
  // the re-solved cut (k_resolve); at kappa 0 and infinity lambda does not depend on
  // the bias, so it cuts where the frozen reading does and differs only in the bias it
  // reports (that of the kept set)
  const bool resolved = (mode.flags & VERKV_STEP_RESOLVED) != 0;
  int team = std::min(L.team, team_size(rows, t.max_n));
  while (team > 1 && team * rows > decide_capacity(t.max_n, team)) --team;
  if (resolved) {
    int cus = 256, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    auto fits = [&](int tm) {
      return tm * rows <= cus * resolve_blocks_per_cu(chunks_of(t.max_n),
                                                      decide_slice_cached(t.max_n, tm));
    };
    while (team > 1 && !fits(team)) --team;
  }
  dc.team = team;
  dc.xcd_map = (team > 1 && rows % 8 == 0) ? 1 : 0;
  dc.team_ws = L.team;
  dc.bprev = reinterpret_cast<double *>(ws + L.bprev);
  dc.xseq = sk.xseq;
  dc.part = reinterpret_cast<double *>(ws + L.part);
  dc.hcnt = reinterpret_cast<uint32_t *>(ws + L.hcnt);
  dc.hbeta = reinterpret_cast<double *>(ws + L.hbeta);
  dc.hV = reinterpret_cast<double *>(ws + L.hV);
  dc.hmax = reinterpret_cast<uint64_t *>(ws + L.hmax);
  dc.wkey = reinterpret_cast<uint64_t *>(ws + L.wkey);
  dc.wlo = reinterpret_cast<uint32_t *>(ws + L.wlo);
  dc.wcount = sk.wcount;
  dc.phase_clock = nullptr;
  dc.resolved = resolved ? 1 : 0;
  dc.gpar = reinterpret_cast<double *>(ws + L.gpar);
#ifdef VERKV_PHASE_TIMING
  if (workspace_bytes >= L.total + (size_t)rows * team * 64 * 8)
    dc.phase_clock = reinterpret_cast<uint64_t *>(ws + L.total);
#endif
  {
    Timed tm(K_DECIDE, stream);
    HIP_TRY(launch_decide(dc, rows, stream), "decide launch");
  }
  if ((rc = launch_pf()) != VERKV_OK) return rc;
  if (resolved) {
    ResolveArgs rv;
    rv.t = t;
    rv.wc = sk.wc;
    rv.cscale = dc.cscale;
    rv.cf0 = sk.cf0;
    rv.r = st->r;
    rv.fbits = sk.fbits;
    rv.kappa = beta;
    rv.eps = eps;
    rv.l = dc.l;
    rv.d_sketch = out->d_sketch;
    rv.beta_star = out->beta_star;
    rv.certified = out->certified;
    rv.kstar = out->kstar;
    rv.gpar = dc.gpar;
    rv.status = dc.status;
    rv.team = dc.team;
    rv.xcd_map = dc.xcd_map;
    rv.team_ws = dc.team_ws;
    rv.xseq = dc.xseq;
    rv.part = dc.part;
    rv.hcnt = dc.hcnt;
    rv.wkey = dc.wkey;
    rv.wlo = dc.wlo;
    rv.wcount = dc.wcount;
    rv.nch_max = dc.nch_max;
    rv.lds_cache = dc.lds_cache;
    Timed tm(K_RESOLVE, stream);
    HIP_TRY(launch_resolve(rv, rows, stream), "resolve launch");
  }

  UnionArgs un;
  un.t = t;
  un.fbits = sk.fbits;
  un.resident = st->resident;
  un.piv_idx = st->piv_idx;
  un.piv_count = st->piv_count;
  un.cap = st->cap;
  un.r = st->r;
  un.wc = sk.wc;
  un.cscale = dc.cscale;
  un.beta_star = out->beta_star;
  un.kappa = beta;
  un.fetch_idx = out->fetch_idx;
  un.fetch_cap = out->fetch_cap;
  un.fetch_count = out->fetch_count;
  un.h2d_count = out->h2d_count;
  un.h2d_idx = reinterpret_cast<int32_t *>(ws + L.h2d);
  un.coef = reinterpret_cast<float *>(ws + L.coef);
  un.params = nullptr;
  un.coef_pass = 0;
  un.slot_of = prefetch && sg.rows > 0 ? reinterpret_cast<const int32_t *>(ws + L.slot_of) : nullptr;
  un.stage_rows = prefetch ? sg.rows : 0;
  un.shdr = prefetch ? reinterpret_cast<uint64_t *>(ws + L.shdr) : nullptr;
  un.ident_ptr = reinterpret_cast<uint64_t>(Vd);
  un.ident_shape = stage_ident(t, bf16, Kd);
  un.h2d_count_ws = reinterpret_cast<int32_t *>(ws + L.h2dc);
  un.stg_cnt = reinterpret_cast<int32_t *>(ws + L.stg);
  un.piv_sched = nullptr;
  un.piv_runs = nullptr;
  un.piv_workers = 0;
  // the estimator coefficients of the resident pivots and the pivot schedule need only
  // the decisions: on the second stream they run beside the list kernel, before the
  // host-row kernel of verkv_refine fills the CUs
  if (mode.side) {
    UnionArgs cf = coef_args(t, st, ws, L, out, units);
    HIP_TRY(hipEventRecord(sd->dec, stream), "hipEventRecord");
    HIP_TRY(hipStreamWaitEvent(sd->s, sd->dec, 0), "hipStreamWaitEvent");
    {
      Timed tm(K_COEF, sd->s);
      HIP_TRY(launch_union(cf, units, sd->s), "pivot coefficient launch");
    }
    // eps_after's terms too: small, and off the chain verkv_refine puts on this stream
    // (the pivot attention, which starts after the list kernel, then the plan)
    if ((rc = launch_after_terms(t, st, out, ws, L, sd->s)) != VERKV_OK) return rc;
  }
  // the list kernel tags entries with the slots the copies filled
  if (prefetch) HIP_TRY(hipStreamWaitEvent(stream, sd->pref, 0), "hipStreamWaitEvent");
  {
    Timed tm(K_UNION, stream);
    HIP_TRY(launch_union(un, units, stream), "union launch");
  }

  return VERKV_OK;
}

static verkv_status refine_impl(const verkv_shape *s, const verkv_state *st, const float *q,
                                const void *K_host, const void *V_host, verkv_step_out *out,
                                void *workspace, size_t workspace_bytes, hipStream_t stream,
                                const StepMode &mode) {
  SeqTable t;
  const void *Kd = nullptr, *Vd = nullptr;
  verkv_status rc = refine_args(s, st, q, K_host, V_host, out, t, &Kd, &Vd);
  if (rc != VERKV_OK) return rc;
  if (!workspace) return VERKV_EINVAL;
  const bool bf16 = s->kv_dtype == VERKV_BF16;
  const DecodeWs L = decode_layout(t, st->cap, bf16, mode.staging);
  if (workspace_bytes < L.total) return VERKV_EWORKSPACE;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  const int units = t.B * t.Hkv;
  const int rows = units * t.G;
  // the caches the next step's staging reads (resolved before anything is enqueued)
  const void *Vs = nullptr, *Ks = nullptr;
  if (mode.side && (rc = prefetch_source(st, L.srows, &Vs, &Ks)) != VERKV_OK) return rc;

  // the resident-pivot side runs on the library's second stream (forked from and joined
  // back into the caller's), or on the caller's stream after the host rows
  Side *sd = nullptr;
  std::unique_lock<std::mutex> lk;
  hipStream_t side = stream;
  if (mode.side) {
    if ((rc = side_for_device(&sd)) != VERKV_OK) return rc;
    lk = std::unique_lock<std::mutex>(sd->mu);
    side = sd->s;
    // fork: the side stream starts where the caller's stream is now
    HIP_TRY(hipEventRecord(sd->fork, stream), "hipEventRecord");
    HIP_TRY(hipStreamWaitEvent(sd->s, sd->fork, 0), "hipStreamWaitEvent");
  }

  // caller's stream: rows F \ S from the host cache
  AttendArgs at;
  at.t = t;
  at.q = q;
  at.m_hat = out->m_hat;
  at.inv_sqrt_d = (float)(1.0 / std::sqrt((double)VERKV_HEAD_DIM));
  at.krows = static_cast<const uint8_t *>(Kd);
  at.vrows = static_cast<const uint8_t *>(Vd);
  at.count = out->h2d_count;
  at.list = reinterpret_cast<const int32_t *>(ws + L.h2d);
  at.coef = nullptr;
  at.cap = st->cap;
  at.part = reinterpret_cast<float *>(ws + L.hpart);
  at.nsplit = L.nsh;
  at.sched = nullptr;
  at.runs = nullptr;
  at.wc = reinterpret_cast<const double *>(ws + L.wc);
  at.cscale = reinterpret_cast<const double *>(ws + L.cscale);
  at.stage = ws + L.stage;
  at.stage_tok = reinterpret_cast<const int32_t *>(ws + L.stage_tok);
  // the slot geometry of this state's prefetch (list entries carry slots only for rows
  // that a prefetch with this geometry staged)
  const StageGeom sg = stage_geom(L.srows, bf16, !st->sketch_exact && st->k_host && st->v_host);
  at.stage_rows = sg.rows;
  at.stage_stride = sg.stride;
  at.stage_kv = sg.kv ? 1 : 0;
  at.stg_cnt = reinterpret_cast<int32_t *>(ws + L.stg);
  {
    Timed tm(K_HOST, stream);
    HIP_TRY(launch_attend(at, units, bf16, true, st->sketch_exact != 0, stream),
            "host attention launch");
  }

  // the estimator coefficients of the resident pivots: on the second stream they were
  // computed by verkv_decode_step; on the caller's stream they are computed here
  const UnionArgs un = coef_args(t, st, ws, L, out, units);
  if (!mode.side) {
    Timed tm(K_COEF, side);
    HIP_TRY(launch_union(un, units, side), "pivot coefficient launch");
  }

  AttendArgs pv;
  pv.t = t;
  pv.q = q;
  pv.m_hat = out->m_hat;
  pv.inv_sqrt_d = at.inv_sqrt_d;
  pv.krows = static_cast<const uint8_t *>(st->piv_k);
  pv.vrows = static_cast<const uint8_t *>(st->piv_v);
  pv.count = st->piv_count;
  pv.list = nullptr;
  pv.coef = reinterpret_cast<const float *>(ws + L.coef);
  pv.cap = st->cap;
  pv.part = reinterpret_cast<float *>(ws + L.ppart);
  pv.nsplit = un.piv_workers;
  pv.sched = un.piv_sched;
  pv.runs = un.piv_runs;
  pv.wc = nullptr;
  pv.cscale = nullptr;
  pv.stage = nullptr;
  pv.stage_tok = nullptr;
  pv.stage_rows = 0;
  pv.stage_stride = 0;
  pv.stage_kv = 0;
  pv.stg_cnt = nullptr;
  {
    Timed tm(K_PIVOT, side);
    HIP_TRY(launch_attend(pv, units, bf16, false, false, side), "pivot attention launch");
  }

  // eps_after's terms: verkv_decode_step put them on the second stream; without it, here
  if (!mode.side && (rc = launch_after_terms(t, st, out, ws, L, side)) != VERKV_OK) return rc;

  // the staging plan of the next step, from this step's list, last on the second stream
  if (Vs) {
    const PrefetchArgs pl = stage_args(t, ws, L, Vs, Ks, bf16, stage_geom(L.srows, bf16, Ks != nullptr));
    Timed tm(K_PLAN, side);
    HIP_TRY(launch_stage_plan(pl, units, side), "staging plan launch");
  }
  // join before the finishing kernel
  if (mode.side) {
    HIP_TRY(hipEventRecord(sd->join, sd->s), "hipEventRecord");
    HIP_TRY(hipStreamWaitEvent(stream, sd->join, 0), "hipStreamWaitEvent");
  }

  FinishArgs fi;
  fi.t = t;
  fi.piv_part = reinterpret_cast<const float *>(ws + L.ppart);
  fi.piv_runs = un.piv_runs;
  fi.host_part = at.part;
  fi.nsh = L.nsh;
  fi.wc = reinterpret_cast<const double *>(ws + L.wc);
  fi.cscale = reinterpret_cast<const double *>(ws + L.cscale);
  fi.r = st->r;
  fi.fbits = reinterpret_cast<const uint32_t *>(ws + L.fbits);
  fi.m_hat = out->m_hat;
  fi.d_sketch = out->d_sketch;
  fi.beta_star = out->beta_star;
  fi.params = reinterpret_cast<const double *>(ws + L.status + 32);   // kappa, l of the step
  fi.after_part = reinterpret_cast<const double *>(ws + L.apart);
  fi.team = L.team;
  fi.eps_after = out->eps_after;
  fi.n_hat = out->n_hat;
  fi.d_hat = out->d_hat;
  fi.o = out->o;
  fi.lse = out->lse;
  {
    Timed tm(K_FINISH, stream);
    HIP_TRY(launch_finish(fi, rows, stream), "finish launch");
  }
  (void)rows;
  return VERKV_OK;
}

verkv_status verkv_decode_step(const verkv_shape *s, const verkv_state *st, const float *q,
                               double beta, double eps, double delta, verkv_step_out *out,
                               void *workspace, size_t workspace_bytes, verkv_stream_t stream) {
  return decode_impl(s, st, q, beta, eps, delta, out, workspace, workspace_bytes,
                     reinterpret_cast<hipStream_t>(stream), StepMode{});
}

verkv_status verkv_decode_step_ex(const verkv_shape *s, const verkv_state *st, const float *q,
                                  double beta, double eps, double delta, verkv_step_out *out,
                                  void *workspace, size_t workspace_bytes, uint32_t flags,
                                  verkv_stream_t stream) {
  if (flags & ~(uint32_t)VERKV_STEP_RESOLVED) return VERKV_EINVAL;
  StepMode mode;
  mode.flags = flags;
  return decode_impl(s, st, q, beta, eps, delta, out, workspace, workspace_bytes,
                     reinterpret_cast<hipStream_t>(stream), mode);
}

verkv_status verkv_refine(const verkv_shape *s, const verkv_state *st, const float *q,
                          const void *K_host, const void *V_host, verkv_step_out *out,
                          void *workspace, size_t workspace_bytes, verkv_stream_t stream) {
  return refine_impl(s, st, q, K_host, V_host, out, workspace, workspace_bytes,
                     reinterpret_cast<hipStream_t>(stream), StepMode{});
}

size_t verkv_noalloc_scratch_bytes(void) { return STATIC_SCRATCH_BYTES; }

verkv_status verkv_step_noalloc(const verkv_shape *s, const verkv_state *st, const float *q,
                                double beta, double eps, double delta, const void *K_host,
                                const void *V_host, verkv_step_out *out, int32_t *status,
                                verkv_stream_t stream_) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  // every argument of both halves is checked before the first launch
  SeqTable t;
  verkv_status rc = decode_args(s, st, q, beta, eps, delta, out, t);
  if (rc != VERKV_OK) return rc;
  const void *Kd = nullptr, *Vd = nullptr;
  if ((rc = refine_args(s, st, q, K_host, V_host, out, t, &Kd, &Vd)) != VERKV_OK) return rc;
  const size_t need = decode_layout(t, st->cap, s->kv_dtype == VERKV_BF16, false).total;
  if (need > STATIC_SCRATCH_BYTES) {
    std::snprintf(g_last_error, sizeof(g_last_error),
                  "this shape needs %zu bytes of scratch; the static array holds %zu", need,
                  STATIC_SCRATCH_BYTES);
    return VERKV_EWORKSPACE;
  }
  uint8_t *ptr = nullptr;
  if ((rc = scratch_for_device(&ptr)) != VERKV_OK) return rc;
  StepMode mode;
  mode.staging = false;
  mode.side = false;
  mode.status = status;
  if ((rc = decode_impl(s, st, q, beta, eps, delta, out, ptr, STATIC_SCRATCH_BYTES, stream, mode)) !=
      VERKV_OK)
    return rc;
  return refine_impl(s, st, q, K_host, V_host, out, ptr, STATIC_SCRATCH_BYTES, stream, mode);
}

verkv_status verkv_check(void *workspace, const verkv_shape *s, int32_t cap, verkv_stream_t stream_) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  SeqTable t;
  verkv_status rc = make_table(s, t);
  if (rc != VERKV_OK) return rc;
  if (!workspace || cap < 1) return VERKV_EINVAL;
  const DecodeWs L = decode_layout(t, cap, s->kv_dtype == VERKV_BF16);
  int32_t *status = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(workspace) + L.status);
  int32_t h = 0;
  HIP_TRY(hipMemcpyAsync(&h, status, sizeof(h), hipMemcpyDeviceToHost, stream), "hipMemcpyAsync");
  HIP_TRY(hipStreamSynchronize(stream), "hipStreamSynchronize");
  if (h == 0) return VERKV_OK;
  const int32_t zero = 0;
  HIP_TRY(hipMemcpyAsync(status, &zero, sizeof(zero), hipMemcpyHostToDevice, stream), "hipMemcpyAsync");
  HIP_TRY(hipStreamSynchronize(stream), "hipStreamSynchronize");
  std::snprintf(g_last_error, sizeof(g_last_error), "kernel flags 0x%x:%s%s", h,
                (h & 4) ? " team barrier timed out;" : "",
                (h & 2) ? " fixed point did not converge;" : "");
  return VERKV_EHIP;
}

int32_t verkv_profile_begin(int32_t max_launches) {
  verkv_profile_end();
  if (max_launches < 1) return VERKV_EINVAL;
  g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
  g_prof.kind.assign((size_t)max_launches, -1);
  for (auto &e : g_prof.ev) {
    hipError_t rc = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
    if (rc != hipSuccess) {
      verkv_profile_end();
      return hip_fail(rc, "hipEventCreate");
    }
  }
  g_prof.used = 0;
  g_prof.on = true;
  return VERKV_OK;
}

int32_t verkv_profile_report(double *total_ms, int32_t *launches, int32_t n_kinds) {
  if (!total_ms || !launches || n_kinds < VERKV_PROFILE_KINDS) return VERKV_EINVAL;
  for (int k = 0; k < VERKV_PROFILE_KINDS; ++k) { total_ms[k] = 0.0; launches[k] = 0; }
  for (size_t i = 0; i < g_prof.used; ++i) {
    if (g_prof.kind[i] < 0) continue;
    HIP_TRY(hipEventSynchronize(g_prof.ev[2 * i + 1]), "hipEventSynchronize");
    float ms = 0.0f;
    HIP_TRY(hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]), "hipEventElapsedTime");
    total_ms[g_prof.kind[i]] += ms;
    launches[g_prof.kind[i]] += 1;
  }
  g_prof.used = 0;
  return VERKV_OK;
}

verkv_status verkv_gather_rows_memcpy(const void *src, size_t row_bytes, const int32_t *idx,
                                      int32_t count, void *dst, int64_t *runs,
                                      verkv_stream_t stream) {
  if (runs) *runs = 0;
  if (!src || !dst || row_bytes == 0 || count < 0 || (count > 0 && !idx)) return VERKV_EINVAL;
  for (int32_t i = 0; i < count; ++i) {
    if (idx[i] < 0 || (i > 0 && idx[i] <= idx[i - 1])) {
      std::snprintf(g_last_error, sizeof(g_last_error), "row list is not ascending at entry %d", (int)i);
      return VERKV_EINVAL;
    }
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint8_t *s8 = static_cast<const uint8_t *>(src);
  uint8_t *d8 = static_cast<uint8_t *>(dst);
  int64_t nrun = 0;
  for (int32_t i = 0; i < count;) {
    int32_t j = i + 1;
    while (j < count && idx[j] == idx[j - 1] + 1) ++j;      // one run of consecutive rows
    HIP_TRY(hipMemcpyAsync(d8 + (size_t)i * row_bytes, s8 + (size_t)idx[i] * row_bytes,
                           (size_t)(j - i) * row_bytes, hipMemcpyHostToDevice, st),
            "hipMemcpyAsync");
    ++nrun;
    i = j;
  }
  if (runs) *runs = nrun;
  return VERKV_OK;
}

void verkv_profile_end(void) {
  for (auto &e : g_prof.ev)
    if (e) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.kind.clear();
  g_prof.used = 0;
  g_prof.on = false;
}

}  // extern "C"
