// A growing cache for gfx950: one decode-time token appended to every sequence of a
// batch.  The pages ("Verify Before You Fetch", picx.dev summary page, "Methodology",
// subsection "POISSONCOMP") compress the cache once, at prefill, and say nothing about
// the tokens decode appends; the reading taken here keeps the prefill's rule:
//   * the appended token n joins the local window: r_n = 1, resident;
//   * the token leaving the window, t = n - n_local (unless it is a sink token), gets
//     eq. (3)'s rule with the prefill's water level c: r_t = min(1, fl(c Q_t)) with
//     Q_t = ceil(tau_t 2^40) (r = 1 / 0 / [Q_t > 0] where the prefill took the "all",
//     "no budget" or "saturated" branch), and, when 0 < r_t < 1, its Bernoulli draw
//     with the Philox counter (t, kv_head, layer, sequence) it would have had at prefill;
//   * with no local window the appended token itself gets the rule and the draw;
//   * the level is not re-solved, so the resident budget grows by r_t per token.
// The pivot list stays ascending: the last n_local entries are the window, so t (when
// it is not kept) is removed by shifting those entries down one place, and n is
// appended.  The pivot K/V rows are stored in the order the pivot-attention schedule
// reads them, which depends on every head's pivot count, so they are copied out in list
// order under the old counts' schedule and back under the new one (the new token's rows
// read from the cache).  If any head's list would exceed the pivot capacity, or the
// state does not match the shape, nothing is changed and the status word says so.
#include "kernels.h"

namespace verkv {

constexpr int AP_NT = 256;
constexpr int PLAN_NT = 1024;

// Per (sequence, KV head): what the append does.  One workgroup: it clears the status
// word, then each thread plans its heads and flags problems there.
__global__ __launch_bounds__(PLAN_NT) void k_append_plan(AppendArgs a) {
  if (threadIdx.x == 0) *a.status = 0;
  __syncthreads();
  const int units = a.t.B * a.t.Hkv;
  for (int u = threadIdx.x; u < units; u += PLAN_NT) {
    const int b = u / a.t.Hkv;
    const int g = u % a.t.Hkv;
    const int n = a.t.s[b].n;
    const int count = a.piv_count[u];
    if (count < 0 || count > a.cap || n + 1 > a.t.s[b].cap) {
      atomicOr(a.status, 16);                    // not a state of this shape
      continue;
    }
    const int64_t tb = tok_base(a.t, b, g);
    const int t = n - a.t.n_local;               // leaves the window (n itself without one)
    const bool rule = a.t.n_sink <= t;
    bool keep = true;
    double rt = 1.0;
    if (rule) {
      const float x = a.tau[tb + t];
      if (!(x >= 0.0f && x <= 1.0f)) {
        atomicOr(a.status, 1);
        continue;
      }
      const double lv = a.level[u];
      const uint64_t q = (uint64_t)ceil((double)x * 0x1.0p40);
      if (lv == LEVEL_ALL) rt = 1.0;
      else if (lv == LEVEL_NONE) rt = 0.0;
      else if (lv == LEVEL_SATURATED) rt = q > 0 ? 1.0 : 0.0;
      else {
        const double cq = lv * (double)q;
        rt = cq >= 1.0 ? 1.0 : cq;
      }
      keep = rt >= 1.0 ||
             (rt > 0.0 && philox_uniform53((uint32_t)t, (uint32_t)g, a.layer, (uint32_t)b, a.seed) < rt);
    }
    int drop = -1, count_new = count + 1, n_in = 1;
    if (rule && t == n) {                        // no window: the new token took the rule
      n_in = keep ? 1 : 0;
      count_new = count + n_in;
    } else if (rule && !keep) {
      drop = count - a.t.n_local;                // t opens the window's run of entries
      count_new = count;
      if (drop < 0 || a.piv_idx[(int64_t)u * a.cap + drop] != t) {
        atomicOr(a.status, 16);
        continue;
      }
    }
    if (count_new > a.cap) atomicOr(a.status, 8);
    a.plan[u] = make_int4(drop, count_new, n_in, count);
    a.plan_r[u] = rt;
  }
}

// r, the resident bits, the pivot list and its count.  One thread per head (the list
// changes in at most n_local + 1 entries).
__global__ __launch_bounds__(AP_NT) void k_append_apply(AppendArgs a) {
  if (*a.status & APPEND_BAD) return;
  const int units = a.t.B * a.t.Hkv;
  const int u = blockIdx.x * AP_NT + threadIdx.x;
  if (u >= units) return;
  const int b = u / a.t.Hkv;
  const int g = u % a.t.Hkv;
  const int n = a.t.s[b].n;
  const int4 pl = a.plan[u];
  const int t = n - a.t.n_local;
  const bool rule = a.t.n_sink <= t;
  double *r = a.r + tok_base(a.t, b, g);
  uint32_t *res = a.resident + word_base(a.t, b, g);
  auto set_bit = [&](int i, bool on) {
    const uint32_t m = 1u << (i & 31);
    res[i >> 5] = on ? (res[i >> 5] | m) : (res[i >> 5] & ~m);
  };
  r[n] = 1.0;
  set_bit(n, true);
  if (rule) {
    r[t] = a.plan_r[u];
    // t == n: the new token itself; otherwise t was in the window and resident
    set_bit(t, t == n ? pl.z != 0 : pl.x < 0);
  }
  int32_t *pidx = a.piv_idx + (int64_t)u * a.cap;
  if (pl.x >= 0)
    for (int p = pl.x; p + 1 < pl.w; ++p) pidx[p] = pidx[p + 1];
  if (pl.z) pidx[pl.y - 1] = n;
  a.piv_count[u] = pl.y;
}

// Pivot K/V rows between the schedule-ordered storage and the workspace (rows in list
// order): out, under the old counts' schedule; in, under the new one, taking each new
// list entry from its old place (or the cache for the new token) and writing zeros to
// the rest of the head's last chunk, as the prefill's gather does.
template <bool IN>
__global__ __launch_bounds__(256) void k_append_copy(AppendArgs a) {
  if (*a.status & APPEND_BAD) return;
  const int unit = blockIdx.y;
  const int b = unit / a.t.Hkv;
  const int g = unit % a.t.Hkv;
  const int4 pl = a.plan[unit];
  const int cnt = IN ? pl.y : pl.w;
  const int lim = IN ? (cnt + PIVOT_CHUNK - 1) / PIVOT_CHUNK * PIVOT_CHUNK : cnt;
  const int p0 = blockIdx.x * GATHER_ROWS;
  if (p0 >= lim) return;
  const int4 *sched = IN ? a.sched_new : a.sched_old;
  const int4 *runs = IN ? a.runs_new : a.runs_old;
  const int4 hdr = sched[2 * a.workers];
  const int64_t NC = hdr.x, P = hdr.y;
  if (NC <= 0 || P <= 0) return;
  const int64_t c_u = runs[unit].z;
  const int per_row = a.row_bytes / 16;
  const int nrow = min(GATHER_ROWS, lim - p0);
  const int64_t list0 = (int64_t)unit * a.cap;
  for (int e = threadIdx.x; e < nrow * per_row; e += blockDim.x) {
    const int p = p0 + e / per_row;
    const int piece = e % per_row;
    const int64_t row = pivot_store_row(c_u, p, NC, P);
    if (row < 0 || row >= a.rows) continue;      // never, for a schedule of these counts
    const int64_t sof = row * a.row_bytes + (int64_t)piece * 16;
    if (!IN) {
      const int64_t dof = (list0 + p) * a.row_bytes + (int64_t)piece * 16;
      *(uint4 *)(a.rows_k + dof) = *(const uint4 *)(a.piv_k + sof);
      *(uint4 *)(a.rows_v + dof) = *(const uint4 *)(a.piv_v + sof);
      continue;
    }
    uint4 kk = make_uint4(0u, 0u, 0u, 0u), vv = kk;
    if (p < cnt) {
      if (pl.z && p == cnt - 1) {                // the appended token, from the cache
        const int64_t so = (tok_base(a.t, b, g) + a.t.s[b].n) * a.row_bytes + (int64_t)piece * 16;
        kk = *(const uint4 *)(a.K_host + so);
        vv = *(const uint4 *)(a.V_host + so);
      } else {
        const int old = (pl.x >= 0 && p >= pl.x) ? p + 1 : p;
        const int64_t so = (list0 + old) * a.row_bytes + (int64_t)piece * 16;
        kk = *(const uint4 *)(a.rows_k + so);
        vv = *(const uint4 *)(a.rows_v + so);
      }
    }
    *(uint4 *)(a.piv_k + sof) = kk;
    *(uint4 *)(a.piv_v + sof) = vv;
  }
}

hipError_t launch_append_plan(const AppendArgs &a, int units, hipStream_t st) {
  (void)units;
  return launch_kernel(k_append_plan, dim3(1), dim3(PLAN_NT), 0, st, a);
}

hipError_t launch_append_apply(const AppendArgs &a, int units, hipStream_t st) {
  return launch_kernel(k_append_apply, dim3((units + AP_NT - 1) / AP_NT), dim3(AP_NT), 0, st, a);
}

hipError_t launch_append_copy(const AppendArgs &a, int units, bool in, hipStream_t st) {
  const int nblk = (a.cap + GATHER_ROWS - 1) / GATHER_ROWS;
  if (in) return launch_kernel(k_append_copy<true>, dim3(nblk, units), dim3(256), 0, st, a);
  return launch_kernel(k_append_copy<false>, dim3(nblk, units), dim3(256), 0, st, a);
}

}  // namespace verkv
