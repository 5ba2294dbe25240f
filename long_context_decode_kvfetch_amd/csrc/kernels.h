// Kernel argument blocks and launchers of the VerKV library (internal).
#pragma once
#include "common.h"
#include <hip/hip_ext.h>

namespace verkv {

struct CompressArgs {
  SeqTable t;
  const float *tau;           // [B][Hkv][n]
  double eta;
  uint64_t seed;
  uint32_t layer;
  double *r;                  // [B][Hkv][n]
  uint32_t *resident;         // [B][Hkv][W]
  int32_t *piv_idx;           // [B][Hkv][cap]
  int32_t *piv_count;         // [B][Hkv]
  int32_t cap;
  uint64_t *keys_a;           // workspace [B][Hkv][n]
  uint64_t *keys_b;           // workspace [B][Hkv][n]
  int32_t *status;            // workspace [0]: error bits, [1]: max pivot count
  double *level;              // [B][Hkv] water level c, or the branch code (null: not kept)
};

// Branch codes kept in verkv_state.level where eq. (3)'s water level is not used.
constexpr double LEVEL_ALL = -1.0;        // every non-forced token has r = 1
constexpr double LEVEL_NONE = -2.0;       // no budget left: r = 0
constexpr double LEVEL_SATURATED = -3.0;  // every positive score saturated: r = [tau > 0]

// One token appended to every sequence of a batch (the growing cache).
struct AppendArgs {
  SeqTable t;                 // lengths before the append (token n_b is appended)
  const float *tau;           // [B][Hkv][cap] scores; the new token's at index n_b
  const double *level;        // [B][Hkv] from PoissonComp
  double *r;                  // [B][Hkv][cap]
  uint32_t *resident;         // [B][Hkv][W]
  int32_t *piv_idx;           // [B][Hkv][cap_piv]
  int32_t *piv_count;         // [B][Hkv]
  int32_t cap;                // pivot capacity
  uint64_t seed;
  uint32_t layer;
  int32_t *status;            // caller's word: 1 tau outside [0, 1], 8 pivot capacity, 16 state
  int4 *plan;                 // workspace [B*Hkv]: {drop position or -1, new count, token n kept, old count}
  double *plan_r;             // workspace [B*Hkv]: r of the token that gets the rule
  // pivot rows, re-laid out in the order of the new counts' schedule
  const uint8_t *K_host, *V_host;   // device views of the cache (the new token's rows)
  uint8_t *piv_k, *piv_v;
  uint8_t *rows_k, *rows_v;   // workspace [B*Hkv][cap_piv][row]: rows in list order
  const int4 *sched_old, *runs_old, *sched_new, *runs_new;
  int32_t workers;
  int32_t row_bytes;
  int64_t rows;               // rows allocated in piv_k / piv_v
};
constexpr int32_t APPEND_BAD = 1 | 8 | 16;

struct GatherArgs {
  SeqTable t;
  const uint8_t *K_host, *V_host;   // device-visible pointers to the pinned host cache
  const int32_t *piv_idx, *piv_count;
  uint8_t *piv_k, *piv_v;           // [pivot rows][128], rows in the pivot schedule's order
  int32_t cap;
  int32_t row_bytes;
  const int4 *sched;                // pivot schedule (header {NC, P} after the worker pairs)
  const int4 *runs;                 // per KV head {first slot, runs, first chunk, 0}
  int32_t workers;                  // worker pairs in `sched`
  int64_t rows;                     // rows allocated in piv_k / piv_v
};

// The pivot-attention schedule (computed by one workgroup).
struct PlanArgs {
  SeqTable t;
  const int32_t *piv_count;
  int32_t cap;
  int32_t workers;
  int4 *sched;               // [2 workers + 1]
  int4 *runs;                // [B][Hkv]
};

// The 2-bit sketch rows of a key cache.
struct QuantArgs {
  const uint8_t *K;          // [rows][128] kv dtype (device-visible)
  uint8_t *out;              // [rows][SKETCH2_ROW_BYTES]
  int64_t rows;              // Hkv * total tokens
};

struct SketchArgs {
  SeqTable t;
  const uint8_t *sketch;      // [B][Hkv][n][128] kv dtype
  const float *q;             // [B][Hq][128]
  double inv_sqrt_d;          // 1/sqrt(128): scores are q.k / sqrt(d)
  double *wc;                 // [B][Hq][n]
  double2 *cstat;             // [B][Hq][nchunks]  (m_c, sum_c)
  const double *r;            // [B][Hkv][n] inclusion probabilities
  double *cf0;                // [B][Hq][nchunks]  sum over L of wc (1 - r): f(0) per chunk
  uint32_t *fbits;            // [B][Hkv][W]  cleared here
  uint32_t *wcount;           // [B][Hq] decision-kernel window counters, cleared here
  double *xseq;               // [B][Hq][xseq_row] team exchange sequence words, cleared here
  int32_t xseq_row;
  int32_t *kstar;             // [B][Hq] cleared here
  int32_t total_blocks;
  int32_t q2;                 // 1: `sketch` holds 2-bit rows (SKETCH2_ROW_BYTES each)
};

struct DecideArgs {
  SeqTable t;
  const double *wc;          // [B][Hq][n]   exp(s - m_chunk)
  const double2 *cstat;      // [B][Hq][nch] (m_chunk, sum over chunk)
  const double *cf0;         // [B][Hq][nch] f(0) per chunk, relative to m_chunk
  double *cscale;            // [B][Hq][nch] out: exp(m_chunk - m_hat)
  const double *r;           // [B][Hkv][n]
  uint32_t *fbits;           // [B][Hkv][W]
  double kappa, eps, l;
  double *m_hat, *d_sketch, *beta_star, *eps_hat;
  uint8_t *certified;
  int32_t *kstar;
  int32_t *status;
  double *params;            // out: kappa, l of this step (read by the finish kernel)
  // team workspace (T workgroups per row)
  int32_t team;
  int32_t xcd_map;           // 1: map the members of a team to one XCD
  int32_t team_ws;           // member stride TW of the exchange slots (team >= launched T)
  double *xseq;              // [rows][2][TW] exchange sequence words (cleared by the sketch kernel)
  double *part;              // [rows][2][TW][PART] member partials
  uint32_t *hcnt;            // [rows][2][TW][NBUCKET] member histograms
  double *hbeta, *hV;
  uint64_t *hmax;
  uint64_t *wkey;            // [rows][WIN] final window
  uint32_t *wlo;
  uint32_t *wcount;          // [rows] (cleared by the sketch kernel)
  uint64_t *phase_clock;     // [rows][T][64] phase timestamps: 32 wall clock, 32 shader clock
                             // (VERKV_PHASE_TIMING builds)
  double *bprev;             // [rows] B* of the last step (Newton start), kept in the workspace
  int32_t nch_max;           // chunk scales held in dynamic LDS
  int32_t lds_cache;         // 1: the launch reserved LDS for the (w, r) slice cache
  int32_t resolved;          // 1: stop after the certificate (k_resolve makes the cut)
  double *gpar;              // [rows][4] out when resolved: V, b1, b2, sqrt(X) of the full L
};

// The cut of eqs. (9)-(10) with the bias re-solved on every candidate set.
struct ResolveArgs {
  SeqTable t;
  const double *wc, *cscale, *cf0, *r;
  uint32_t *fbits;
  double kappa, eps, l;
  const double *d_sketch;
  double *beta_star;         // in: bias of the full L; out: bias of the kept set
  const uint8_t *certified;
  int32_t *kstar;
  const double *gpar;        // [rows][4] V, b1, b2 and sqrt(X) of the full L (from k_decide)
  int32_t *status;
  int32_t team, xcd_map, team_ws;
  double *xseq, *part;
  uint32_t *hcnt;
  uint64_t *wkey;
  uint32_t *wlo;
  uint32_t *wcount;
  int32_t nch_max, lds_cache;
};

struct AfterArgs {
  SeqTable t;
  const double *wc, *cscale, *r;
  const uint32_t *fbits;
  const double *beta_star;
  const double *params;      // kappa, l written by the decision kernel
  int32_t team;
  double *part;              // [rows][T][8]
};

struct UnionArgs {
  SeqTable t;
  const uint32_t *fbits, *resident;
  const int32_t *piv_idx, *piv_count;
  int32_t cap;
  const double *r, *wc, *cscale, *beta_star;
  double kappa;
  int32_t *fetch_idx;
  int32_t fetch_cap;
  int32_t *fetch_count, *h2d_count;
  int32_t *h2d_idx;          // [B][Hkv][n]
  float *coef;               // [B][Hkv][cap][G]
  int32_t coef_pass;         // 0: fetch lists (grid y = 1); 1: pivot coefficients
  const double *params;      // coefficient pass: params[0] = kappa of the step (device)
  const int32_t *slot_of;    // lists: [B][Hkv][cap] staging slot of each token (-1: none),
                             //   or null without staging
  int32_t stage_rows;        // lists: staging slots per KV head
  uint64_t *shdr;            // lists: staging header to publish (null without a prefetch)
  uint64_t ident_ptr, ident_shape;
  int32_t *h2d_count_ws;     // lists: [B][Hkv] |F \ S| kept in the workspace for the next step
  int32_t *stg_cnt;          // lists: [B][Hkv] staged-row counters of the host-row kernel, cleared
  // coefficient pass: the work schedule of the pivot attention (one extra workgroup)
  int4 *piv_sched;           // [2 PIVOT_WORKERS + 1] per worker: first run, chunks after it
  int4 *piv_runs;            // [B][Hkv] first partial slot, partials, first chunk, 0
  int32_t piv_workers;       // workers the pivot attention launches
};

// Cross-step staging of host rows (k_prefetch.hip).  A slot keeps its row from step to
// step; each step makes the tokens of the first stage_rows entries of the previous step's
// host-row list resident, reading only the rows not yet staged over the host link, into
// slots whose tokens that list no longer holds.  slot_of and stage_tok map tokens to
// slots and back; a pair that does not agree is not a staged row.  The plan reads the
// list of the step that just ran (prev_list, prev_count: that step's list and count).
struct PrefetchArgs {
  SeqTable t;
  const int32_t *prev_list;  // [B][Hkv][n] entries of the previous list (token | slot + 1 above tok_bits)
  const int32_t *prev_count; // [B][Hkv]
  const uint8_t *vrows;      // host value cache (device view) [B][Hkv][n][128]
  const uint8_t *krows;      // host key cache (device view), staged beside the values when
                             //   the sketch is not exact; null: values only
  uint8_t *stage;            // [B*Hkv][stage_rows] slots of stage_stride bytes: the value
                             //   row, then (krows set) the key row
  int32_t *stage_tok;        // [B*Hkv][stage_rows] token each slot holds, -1 if none
  int32_t *slot_of;          // [B][Hkv][cap] slot holding each token, -1 if none
  int32_t *pf_new;           // [B*Hkv][stage_rows] plan: the tokens to bring in, in list order
  int32_t *pf_slot;          // [B*Hkv][stage_rows] plan: the slot each of them takes
  int32_t *pf_count;         // [B*Hkv] plan: how many
  uint64_t *shdr;            // staging header (STAGE_HDR_WORDS)
  uint64_t ident_ptr;        // identity of the cache the staged rows come from: the host
  uint64_t ident_shape;      //   value cache's device address and a hash of the shape
  int32_t stage_rows;
  int32_t stage_stride;      // bytes per slot: one row, or two with krows
};

struct AttendArgs {
  SeqTable t;
  const float *q;            // [B][Hq][128]
  const double *m_hat;       // [B][Hq]
  float inv_sqrt_d;
  const uint8_t *krows;      // pivots [rows][128] in schedule order, or host cache [B][Hkv][n][128]
  const uint8_t *vrows;
  const int32_t *count;      // [B][Hkv] rows in the list
  const int32_t *list;       // host source: [B][Hkv][n] token ids; pivots: null
  const float *coef;         // pivots: [B][Hkv][cap][G]; host: null (coefficient 1)
  int32_t cap;
  float *part;               // host: [B][Hkv][nsplit][G][129]; pivots: [slots][G][129]
  int32_t nsplit;            // host: splits per KV head
  const int4 *sched;         // pivots: per-worker schedule from the coefficient pass
  const int4 *runs;          // pivots: per KV head first slot, partials, first chunk
  const double *wc;          // host source with exact sketch: weights w_hat = wc * cscale
  const double *cscale;
  const uint8_t *stage;      // host source: staged value rows [B*Hkv][stage_rows][stride]
  const int32_t *stage_tok;  //   and their tokens (a list entry's slot is checked against it)
  int32_t stage_rows;
  int32_t stage_stride;      // bytes per slot (the value row first)
  int32_t stage_kv;          // 1: a slot also holds the key row, after the value row
  int32_t *stg_cnt;          // host source: [B][Hkv] rows taken from the staging area (added to)
};

struct FinishArgs {
  SeqTable t;
  const float *piv_part;     // [slots][G][129] partials of the resident pivots
  const int4 *piv_runs;      // [B][Hkv] first slot and number of pivot partials (.x, .y)
  const float *host_part;    // [B][Hkv][nsh][G][129]
  int32_t nsh;
  const double *wc, *cscale, *r;
  const uint32_t *fbits;
  const double *m_hat, *d_sketch, *beta_star;
  const double *params;      // kappa, l written by the decision kernel
  const double *after_part;  // [rows][T][8] from k_after
  int32_t team;
  double *eps_after;
  float *n_hat, *d_hat, *o, *lse;
};

constexpr int NBUCKET = 512;     // digit buckets of the k* search (9-bit digits)
constexpr int PART = 16;         // doubles per team member in an exchange slot
constexpr int TEAM_MAX = 16;     // workgroups per query row in the decision kernel
constexpr int DECIDE_THREADS = 512;
constexpr int TEAM_MIN_TOKENS = 2048;   // tokens per team member, at least
constexpr int WIN = 512;         // final window of the k* search
constexpr int GATHER_ROWS = 64;   // pivot rows per gather workgroup
constexpr int STAGE_SLOTS_DEFAULT = 8192;  // staged rows per KV head by default (at most),
constexpr int STAGE_ROWS_TOTAL = 65536;    // and at most this many over all KV heads
// Staging header words: [0] magic, [1] [2] the cache whose rows the maps hold (published
// by the list kernel); [3] [4] the cache the pending plan was made for, [5] its magic
// (written by the plan); [6] 1 when this step's copies ran (written by the copies).
constexpr int STAGE_HDR_WORDS = 8;
constexpr uint64_t STAGE_MAGIC = 0x7665726b76535447ull;
constexpr uint64_t PLAN_MAGIC = 0x7665726b76504c4eull;
constexpr int SKETCH2_ROW_BYTES = 64;   // a 2-bit sketch row: 32 B of codes, 8 float32
constexpr int PIVOT_CHUNK = 32;   // pivot rows per schedule chunk (whole row batches)
constexpr int PIVOT_WORKERS = 768;  // persistent pivot-attention workgroups (3 per CU)

// Where pivot row p of KV head u is stored: the schedule gives worker w of P the global
// chunks [floor(w NC / P), floor((w + 1) NC / P)); the i-th of them is stored as block
// i P + w (PIVOT_CHUNK rows), so the workers, which advance through their chunks at the
// same pace, read one moving window of memory together.  c_u is the head's first chunk.
__host__ __device__ inline int64_t pivot_store_row(int64_t c_u, int p, int64_t NC, int64_t P) {
  const int64_t c = c_u + p / PIVOT_CHUNK;
  const int64_t w = ((c + 1) * P - 1) / NC;
  const int64_t i = c - w * NC / P;
  return (i * P + w) * PIVOT_CHUNK + p % PIVOT_CHUNK;
}

// Timing of the next launch: when `start` is set, the launcher hands the pair to
// hipExtLaunchKernel, which stamps them from the dispatch packet itself (kernel
// execution time, without the gap before the dispatch), and marks them used.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
extern thread_local LaunchEvents g_launch_ev;

template <typename F, typename... Args>
inline hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t st,
                                Args... args) {
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, g_launch_ev.start, g_launch_ev.stop, 0,
                        args...);
  if (g_launch_ev.start) g_launch_ev.used = true;
  return hipGetLastError();
}

// every argument block is passed by value and must fit the kernel argument segment
static_assert(sizeof(CompressArgs) <= 4096 && sizeof(AppendArgs) <= 4096 && sizeof(GatherArgs) <= 4096 && sizeof(PlanArgs) <= 4096 &&
                  sizeof(SketchArgs) <= 4096 && sizeof(DecideArgs) <= 4096 && sizeof(AfterArgs) <= 4096 &&
                  sizeof(UnionArgs) <= 4096 && sizeof(PrefetchArgs) <= 4096 && sizeof(AttendArgs) <= 4096 &&
                  sizeof(FinishArgs) <= 4096 && sizeof(ResolveArgs) <= 4096,
              "kernel arguments exceed 4 KiB");

hipError_t launch_poissoncomp(const CompressArgs &a, int units, hipStream_t st);
hipError_t launch_append_plan(const AppendArgs &a, int units, hipStream_t st);
hipError_t launch_append_copy(const AppendArgs &a, int units, bool in, hipStream_t st);
hipError_t launch_append_apply(const AppendArgs &a, int units, hipStream_t st);
hipError_t launch_gather_pivots(const GatherArgs &a, int units, hipStream_t st);
hipError_t launch_pivot_schedule(const PlanArgs &a, hipStream_t st);
hipError_t launch_sketch(const SketchArgs &a, bool bf16, hipStream_t st);
hipError_t launch_quant_sketch(const QuantArgs &a, bool bf16, hipStream_t st);
hipError_t launch_decide(DecideArgs &a, int rows, hipStream_t st);
hipError_t launch_union(const UnionArgs &a, int units, hipStream_t st);
hipError_t launch_attend(const AttendArgs &a, int units, bool bf16, bool host, bool exact,
                         hipStream_t st);
hipError_t launch_after(const AfterArgs &a, int rows, hipStream_t st);
hipError_t launch_resolve(ResolveArgs &a, int rows, hipStream_t st);
int resolve_blocks_per_cu(int nch_max, bool slice_cache);
hipError_t launch_finish(const FinishArgs &a, int rows, hipStream_t st);
hipError_t launch_stage_plan(const PrefetchArgs &a, int units, hipStream_t st);
hipError_t launch_stage_fetch(const PrefetchArgs &a, int units, bool bf16, hipStream_t st);
int decide_blocks_per_cu(int max_n, int team);
bool decide_slice_cached(int max_n, int team);

}  // namespace verkv
