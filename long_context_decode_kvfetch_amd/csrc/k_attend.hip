// Attention partials over a list of cache rows for gfx950: the estimator of
// "Verify Before You Fetch" (picx.dev summary page, Definition 2 / eq. 5, extended to
// the numerator N as the "Theoretical Foundation" section describes):
//   D_hat = sum_{H u F} w_i + sum_{S \ F} (lambda_i / r_i) w_i,  N_hat likewise with w_i v_i,
//   w_i = exp(q.k_i / sqrt(d) - m_hat)  (true keys, shifted by the largest sketch score).
// Two sources share one kernel body:
//   * resident pivots H u S (device rows, coefficient from the decision kernels): the
//     HBM stream of every decode step;
//   * rows F \ S read straight from the pinned host cache (zero-copy loads over the
//     host link, coefficient 1): KVFetch step 5.  When the sketch is exact (its rows
//     are the keys) the weights of these rows are the float64 sketch weights of step 1
//     and only the value rows cross the host link.
// Each lane owns a 16-byte slice of a K row and of the matching V row; G query rows
// stay in registers; scores are reduced across the lanes of a row with DPP; no MFMA
// (one to eight query rows per KV head is far too thin for a matrix core).  m_hat is
// known from the sketch pass, so no running maximum is needed.  Every workgroup writes
// its partial (N[G][128], D[G]) so the finishing kernel sums a fixed set in a fixed order.
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace verkv {

constexpr int AT_NT = 256;
constexpr int AT_NW = AT_NT / WAVE;

template <bool BF16, int G, bool HOST, bool EXACT>
__global__ __launch_bounds__(AT_NT) void k_attend(AttendArgs a) {
  using RS = RowSlice<BF16>;
  constexpr int EPL = RS::EPL;
  constexpr int LPT = D / EPL;
  constexpr int TPW = WAVE / LPT;
  constexpr int STEP = AT_NW * TPW;          // rows per workgroup iteration
  constexpr int U = 2;                       // row groups per batch (two batches in flight)
  constexpr int ROW_BYTES = D * (BF16 ? 2 : 4);
  constexpr int PS = D + 1;

  __shared__ float s_acc[AT_NW][TPW][G][D];
  __shared__ float s_den[AT_NW][TPW][G];

  const int unit = blockIdx.y;
  const int split = blockIdx.x;
  const int b = unit / a.t.Hkv;
  const int g = unit % a.t.Hkv;
  const int Hq = a.t.Hkv * G;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wv = threadIdx.x / WAVE;
  const int sub = lane % LPT;
  const int grp = lane / LPT;
  const int d0 = sub * EPL;

  // the list in batches of STEP * U consecutive entries, dealt round-robin to the
  // workgroups of the head: the staged rows (the list's first entries) and the rows
  // read over the host link are spread evenly over the workgroups
  const int cnt = HOST ? a.count[unit] : min(a.count[unit], a.cap);
  const int p1 = cnt;

  float qf[G][EPL];
  float mh[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int64_t qrow = (int64_t)b * Hq + g * G + j;
    const float *qr = a.q + qrow * D + d0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[j][e] = qr[e] * a.inv_sqrt_d;
    mh[j] = (float)a.m_hat[qrow];
  }

  float acc[G][EPL];
  float den[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    den[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.0f;
  }

  const int64_t src_base = HOST ? tok_base(a.t, b, g) : (int64_t)unit * a.cap;
  const int32_t *list = HOST ? a.list + tok_base(a.t, b, g) : nullptr;
  (void)list;
  // the staging area: rows of this cache kept across steps, and the token of each slot
  const uint8_t *stage = a.stage;
  const int32_t *stage_tok = a.stage_tok;
  (void)stage;
  (void)stage_tok;
  const int64_t slice = (int64_t)d0 * (BF16 ? 2 : 4);

  int staged_n = 0;                          // rows this lane group took from the staging area
  // Rows go in batches of STEP * U; the loads of the next batch (and, for pivots, its
  // coefficients) are issued before the current batch is reduced, so every wave keeps
  // a batch in flight while it computes.
  struct Batch {
    uint4 kr[U], vr[U];
    int pp[U], tk[U];
    float cc[U][G];
  };
  auto issue = [&](int base, Batch &bt) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = base + u * STEP + wv * TPW + grp;
      bt.pp[u] = p;
      bt.tk[u] = 0;
      if (p < p1) {
        int tok = p;
        const uint8_t *vsrc = nullptr;
        const uint8_t *ksrc = nullptr;
        if constexpr (HOST) {
          // a list entry is token | (staging slot + 1) << tok_bits; the slot's rows
          // are used when the slot holds this token
          const int32_t e = list[p];
          tok = entry_token(e, a.t.tok_bits);
          const int slot = entry_slot(e, a.t.tok_bits);
          if (slot >= 0 && slot < a.stage_rows && stage_tok[(int64_t)unit * a.stage_rows + slot] == tok) {
            vsrc = stage + ((int64_t)unit * a.stage_rows + slot) * a.stage_stride + slice;
            if (!EXACT && a.stage_kv) ksrc = vsrc + ROW_BYTES;
            staged_n += sub == 0 ? 1 : 0;
          }
        }
        bt.tk[u] = tok;
        const int64_t rowi = src_base + tok;
        if (!EXACT) {
          if (!ksrc) ksrc = a.krows + rowi * ROW_BYTES + slice;
          bt.kr[u] = *(const uint4 *)ksrc;
        }
        if (!vsrc) vsrc = a.vrows + rowi * ROW_BYTES + slice;
        bt.vr[u] = *(const uint4 *)vsrc;
        if constexpr (!HOST) {
          // the row's G coefficients are contiguous ([unit][cap][G]): vector loads
          const float *cp = a.coef + ((int64_t)unit * a.cap + p) * G;
          if constexpr (G % 4 == 0) {
#pragma unroll
            for (int j4 = 0; j4 < G; j4 += 4) {
              const float4 c4 = *(const float4 *)(cp + j4);
              bt.cc[u][j4] = c4.x; bt.cc[u][j4 + 1] = c4.y; bt.cc[u][j4 + 2] = c4.z; bt.cc[u][j4 + 3] = c4.w;
            }
          } else {
#pragma unroll
            for (int j = 0; j < G; ++j) bt.cc[u][j] = cp[j];
          }
        }
      } else {
        bt.kr[u] = make_uint4(0, 0, 0, 0);
        bt.vr[u] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < G; ++j) bt.cc[u][j] = 0.0f;
      }
    }
  };
  auto consume = [&](const Batch &bt) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float w[G];
      if constexpr (EXACT) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const int h = g * G + j;
          double wd = 0.0;
          if (bt.pp[u] < p1)
            wd = a.wc[row_tok_base(a.t, b, h) + bt.tk[u]] *
                 a.cscale[row_chunk_base(a.t, b, h) + bt.tk[u] / SKETCH_CHUNK];
          w[j] = (float)wd;
        }
      } else {
        float x[EPL];
        RS::widen(bt.kr[u], x);
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float dot = 0.0f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) dot = fmaf(qf[j][e], x[e], dot);
          dot = sum16(dot);
          if (LPT == 32) dot += shfl_xor_f(dot, 16);
          w[j] = (bt.pp[u] < p1) ? __expf(dot - mh[j]) : 0.0f;
          if constexpr (!HOST) w[j] *= bt.cc[u][j];
        }
      }
      float v[EPL];
      RS::widen(bt.vr[u], v);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        den[j] += w[j];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(w[j], v[e], acc[j][e]);
      }
    }
  };
  constexpr int SU = STEP * U;
  const int stride = a.nsplit * SU;
  Batch A, B;
  int base = split * SU;
  if (base < p1) issue(base, A);
  while (base < p1) {
    if (base + stride < p1) issue(base + stride, B);
    consume(A);
    base += stride;
    if (base >= p1) break;
    if (base + stride < p1) issue(base + stride, A);
    consume(B);
    base += stride;
  }

  if constexpr (HOST) {                      // staged rows of this wave, for the step's count
    const int64_t w = wave_sum_i64(staged_n);
    if (lane == 0 && w > 0 && a.stg_cnt) atomicAdd(&a.stg_cnt[unit], (int32_t)w);
  }
  (void)staged_n;
  // every row group of every wave leaves its partial in LDS; each output element is
  // then summed over the AT_NW x TPW groups in a fixed order
  if (sub == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) s_den[wv][grp][j] = den[j];
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_acc[wv][grp][j][d0 + e] = acc[j][e];
  }
  __syncthreads();
  float *out = a.part + ((int64_t)unit * a.nsplit + split) * G * PS;
  for (int t = threadIdx.x; t < G * PS; t += AT_NT) {
    const int j = t / PS, d = t % PS;
    float s = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < AT_NW; ++w2)
#pragma unroll
      for (int r2 = 0; r2 < TPW; ++r2) s += (d < D) ? s_acc[w2][r2][j][d] : s_den[w2][r2][j];
    out[t] = s;
  }
}

template <bool BF16, int G, bool HOST, bool EXACT>
static hipError_t launch_attend_t(const AttendArgs &a, int units, hipStream_t st) {
  return launch_kernel(k_attend<BF16, G, HOST, EXACT>, dim3(a.nsplit, units), dim3(AT_NT), 0, st, a);
}

// ------------------------------------------------------------------ resident pivots, persistent
// The same partials as k_attend over the resident pivots, from workgroups that stay
// resident and share the rows evenly: worker w takes the chunks the coefficient pass
// scheduled for it (consecutive chunks of PIVOT_CHUNK rows, possibly over several KV
// heads) and streams them through two alternating row batches: while one batch is
// reduced, the loads of the next are in flight, also across the end of a run (the
// worker's rows of one KV head), whose partial goes to the slot the schedule gives it.
// An issue cursor walks the runs one batch ahead of the reduction; each batch carries
// its run's head, slot and first/last flags.  The worker's first chunk is stored as
// block w, so its first batch is loaded before the schedule is read.  The query rows of
// the first run are loaded before the first rows' coefficients, those of the second run
// (named in the schedule) are staged in LDS at the start, so a run change does not wait
// behind rows in flight.  One row group per batch (a quarter of a 32-row chunk per
// workgroup): on MI355X more rows in flight per wave (two or four row groups, three
// batches in the ring, or four workers per CU) made the stream slower, not faster.  The
// K/V rows are read once per step, so they are loaded non-temporally (streaming cache
// policy): 30.7 -> 28.2 us on the 16-sequence batch.
//
// With four query rows and 16 lanes per key row (bf16) the scores are reduce-scattered:
// after five DPP adds lane s of a row holds the full q.k of query row 2 s[3] + s[2], each
// lane takes exp for that one row and the four weights are broadcast back over the row.
constexpr int PIV_U = 1;           // row groups per batch of a pivot worker

template <bool BF16, int G>
__global__ __launch_bounds__(AT_NT) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_attend_piv(AttendArgs a) {
  using RS = RowSlice<BF16>;
  constexpr int EPL = RS::EPL;
  constexpr int LPT = D / EPL;
  constexpr int TPW = WAVE / LPT;
  constexpr int STEP = AT_NW * TPW;
  constexpr int U = PIV_U;
  constexpr int SU = STEP * U;
  constexpr int ROW_BYTES = D * (BF16 ? 2 : 4);
  constexpr int PS = D + 1;
  constexpr int R = PIVOT_CHUNK;
  constexpr bool RS4 = (G == 4 && LPT == 16);    // reduce-scattered scores
  constexpr int NC = RS4 ? 1 : G;                // coefficients held per lane and row
  constexpr float LOG2E = 1.4426950408889634f;

  __shared__ float s_acc[AT_NW][TPW][G][D];
  __shared__ float s_den[AT_NW][TPW][G];
  __shared__ float s_q2[G][D];                   // second run: scaled query rows
  __shared__ float s_m2[G];                      //   and m_hat log2(e)

  const int Hq = a.t.Hkv * G;
  const int units = a.t.B * a.t.Hkv;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wv = threadIdx.x / WAVE;
  const int sub = lane % LPT;
  const int grp = lane / LPT;
  const int d0 = sub * EPL;
  const int64_t slice = (int64_t)d0 * (BF16 ? 2 : 4);
  const int myrow = RS4 ? 2 * ((sub >> 3) & 1) + ((sub >> 2) & 1) : 0;   // query row of this lane
  const int nslots = a.nsplit + units;
  const int PW = a.sched[2 * a.nsplit].y;          // workers P the rows were stored for
  const float qscale = a.inv_sqrt_d * LOG2E;

  // a batch: the loads of SU rows of one run and what the reduction needs to place them
  struct Batch {
    uint4 kr[U], vr[U];
    float cc[U][NC];
    int base, p1;                // first row of the batch, end row of its run
    int unit, slot, run;         // run's KV head, partial slot, index among the worker's runs
    bool first, last, live;      // first / last batch of its run; false past the worker's rows
  };
  // every lane loads a row (rows past the run's end repeat an in-bounds row and get
  // weight 0), so no register is written while a load into it may be in flight.  K and V
  // rows are stored in schedule order: row p of a run that starts at row q0 and at the
  // worker's i0-th chunk is in block (i0 + (p - q0) / PIVOT_CHUNK) P + w; the
  // coefficients keep the [head][cap] order.
  auto issue = [&](int unit, int base, int p1, int i0, int q0, Batch &bt, bool kv) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = base + u * STEP + wv * TPW + grp;
      const int pc = min(max(min(p, p1 - 1), 0), a.cap - 1);
      if (kv) {
        const int64_t ich = i0 + (pc - q0) / PIVOT_CHUNK;
        const int64_t srow = (ich * PW + blockIdx.x) * PIVOT_CHUNK + (pc & (PIVOT_CHUNK - 1));
        bt.kr[u] = load_stream16(a.krows + srow * ROW_BYTES + slice);
        bt.vr[u] = load_stream16(a.vrows + srow * ROW_BYTES + slice);
      }
      const float *cp = a.coef + ((int64_t)unit * a.cap + pc) * G;
      if constexpr (RS4) {
        bt.cc[u][0] = cp[myrow];
      } else if constexpr (G % 4 == 0) {
#pragma unroll
        for (int j4 = 0; j4 < G; j4 += 4) {
          const float4 c4 = *(const float4 *)(cp + j4);
          bt.cc[u][j4] = c4.x; bt.cc[u][j4 + 1] = c4.y; bt.cc[u][j4 + 2] = c4.z; bt.cc[u][j4 + 3] = c4.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < G; ++j) bt.cc[u][j] = cp[j];
      }
    }
    bt.base = base;
    bt.p1 = p1;
  };

  // query slices pre-scaled by log2(e) / sqrt(d), so a weight is exp2(q.k - m_hat log2 e)
  float qf[G][EPL], mh[G], mh_mine = 0.0f;
  float acc[G][EPL], den[G];
  auto load_q = [&](int unit) {                    // from memory
    const int b = unit / a.t.Hkv, g = unit % a.t.Hkv;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int64_t qrow = (int64_t)b * Hq + g * G + j;
      const float *qr = a.q + qrow * D + d0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[j][e] = qr[e] * qscale;
      mh[j] = (float)(a.m_hat[qrow] * (double)LOG2E);
    }
  };
  auto load_q_lds = [&]() {                        // the second run's, staged at the start
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[j][e] = s_q2[j][d0 + e];
      mh[j] = s_m2[j];
    }
  };
  auto reset = [&]() {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      den[j] = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] = 0.0f;
    }
    if constexpr (RS4) mh_mine = myrow == 0 ? mh[0] : myrow == 1 ? mh[1] : myrow == 2 ? mh[2] : mh[3];
  };
  auto consume = [&](const Batch &bt) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = bt.base + u * STEP + wv * TPW + grp < bt.p1;
      float x[EPL], v[EPL], w[G];
      RS::widen(bt.kr[u], x);
      float dp[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = fmaf(qf[j][e], x[e], dot);
        dp[j] = dot;
      }
      if constexpr (RS4) {
        const bool b3 = (sub >> 3) & 1, b2 = (sub >> 2) & 1;
        float k0 = b3 ? dp[2] : dp[0], k1 = b3 ? dp[3] : dp[1];
        const float s0 = b3 ? dp[0] : dp[2], s1 = b3 ? dp[1] : dp[3];
        k0 += dpp_f<DPP_ROR8>(s0);
        k1 += dpp_f<DPP_ROR8>(s1);
        float k = b2 ? k1 : k0;
        const float o = b2 ? k0 : k1;
        k += dpp_f<DPP_HALF_MIRROR>(o);
        k += dpp_f<DPP_XOR1>(k);
        k += dpp_f<DPP_XOR2>(k);
        float wm = exp2f(k - mh_mine) * bt.cc[u][0];
        wm = valid ? wm : 0.0f;
        // query row j is held by lane 4 j of the row
        w[0] = dpp_f<DPP_ROW_BCAST0 + 0>(wm);
        w[1] = dpp_f<DPP_ROW_BCAST0 + 4>(wm);
        w[2] = dpp_f<DPP_ROW_BCAST0 + 8>(wm);
        w[3] = dpp_f<DPP_ROW_BCAST0 + 12>(wm);
      } else {
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float dot = sum16(dp[j]);
          if (LPT == 32) dot += shfl_xor_f(dot, 16);
          w[j] = valid ? exp2f(dot - mh[j]) * bt.cc[u][j] : 0.0f;
        }
      }
      RS::widen(bt.vr[u], v);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        den[j] += w[j];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(w[j], v[e], acc[j][e]);
      }
    }
  };
  auto epilogue = [&](int slot) {
    if (sub == 0) {
#pragma unroll
      for (int jj = 0; jj < G; ++jj) s_den[wv][grp][jj] = den[jj];
    }
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wv][grp][jj][d0 + e] = acc[jj][e];
    }
    __syncthreads();
    float *out = a.part + (int64_t)slot * G * PS;
    for (int t = threadIdx.x; t < G * PS; t += AT_NT) {
      const int jj = t / PS, d = t % PS;
      float sm = 0.0f;
#pragma unroll
      for (int w2 = 0; w2 < AT_NW; ++w2)
#pragma unroll
        for (int r2 = 0; r2 < TPW; ++r2) sm += (d < D) ? s_acc[w2][r2][jj][d] : s_den[w2][r2][jj];
      out[t] = sm;
    }
    __syncthreads();
  };

  // The first batch is the first rows of the worker's first chunk, stored as block
  // blockIdx.x (schedule order, i = 0): its K/V loads leave before the schedule is read.
  // Rows past a head's last pivot in its last chunk hold zeros (written by the gather),
  // so a row of weight 0 there adds nothing.  Block blockIdx.x < nsplit <= the workers
  // the rows are sized for, so the loads stay inside the buffers for any schedule.
  Batch A, B;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t srow = (int64_t)blockIdx.x * PIVOT_CHUNK + u * STEP + wv * TPW + grp;
    A.kr[u] = load_stream16(a.krows + srow * ROW_BYTES + slice);
    A.vr[u] = load_stream16(a.vrows + srow * ROW_BYTES + slice);
  }
  asm volatile("" ::: "memory");                   // keep them ahead of the schedule read

  // this worker's first run {head, first row, end row, slot} and, queued, its second
  // one {head, end row, slot, chunks left after it}
  const int4 f0 = a.sched[2 * blockIdx.x];
  const int4 f1 = a.sched[2 * blockIdx.x + 1];
  if (!(f0.x >= 0 && f0.x < units && f0.y >= 0 && f0.y < f0.z && f0.z <= a.cap && f0.w >= 0 &&
        f0.w < nslots && PW > (int)blockIdx.x && PW <= a.nsplit))
    return;                                        // no rows for this worker
  int q_unit = f1.x, q_p1 = f1.y, q_slot = f1.z, q_left = f1.w, left = 0;
  if (q_unit < 0) {
    left = q_left;                                 // chunks after the first run, heads unknown
  } else if (!(q_unit < units && q_p1 > 0 && q_p1 <= a.cap && q_slot >= 0 && q_slot < nslots)) {
    q_unit = -1;
    q_left = 0;
  }
  const bool staged = q_unit >= 0;                 // run 1's queries come from LDS

  // the issue cursor: the run and row of the next batch to load
  int iu = f0.x, ib = f0.y, ip1 = f0.z, isl = f0.w, ii0 = 0, iq0 = f0.y, irun = 0;
  bool ifirst = true, idone = false;
  auto issue_next = [&](Batch &bt, bool kv) {
    issue(iu, ib, ip1, ii0, iq0, bt, kv);          // weight-0 rows once the worker is done
    bt.unit = iu;
    bt.slot = isl;
    bt.run = irun;
    bt.first = ifirst;
    bt.last = ib + SU >= ip1;
    bt.live = !idone;
    ifirst = false;
    if (idone) return;
    ib += SU;
    if (ib < ip1) return;
    const int run_end_i0 = ii0 + (ip1 - iq0 + R - 1) / R;
    bool more = false;
    if (q_unit >= 0) {                             // the queued second run
      iu = q_unit;
      ip1 = q_p1;
      isl = q_slot;
      left = q_left;
      q_unit = -1;
      more = true;
    } else if (left > 0) {
      // a third run or later, or a head without pivots in between: read the heads
      for (int u2 = iu + 1; u2 < units; ++u2) {
        const int c = min(a.count[u2], a.cap);
        if (c <= 0) continue;
        const int sl = a.runs[u2].x;
        if (sl >= 0 && sl < nslots) {
          const int take = min((c + R - 1) / R, left);
          left -= take;
          iu = u2;
          ip1 = min(c, take * R);
          isl = sl;
          more = true;
        }
        break;
      }
    }
    if (!more) {
      idone = true;
      ib = ip1;                                    // later batches: weight-0 rows of this run
      return;
    }
    ib = 0;
    ii0 = run_end_i0;
    iq0 = 0;
    ++irun;
    ifirst = true;
  };

  // the queries of the first run, and those of the second run (staged in LDS), are
  // loaded before the first rows: a wait for them then never covers rows in flight
  constexpr int Q2N = (G * D + AT_NT - 1) / AT_NT;
  float q2v[Q2N];
  double m2v = 0.0;
  if (staged) {
    const int b2 = f1.x / a.t.Hkv, g2 = f1.x % a.t.Hkv;
#pragma unroll
    for (int k = 0; k < Q2N; ++k) {
      const int t = threadIdx.x + k * AT_NT;
      q2v[k] = t < G * D ? a.q[((int64_t)b2 * Hq + g2 * G + t / D) * D + t % D] : 0.0f;
    }
    if (threadIdx.x < G) m2v = a.m_hat[(int64_t)b2 * Hq + g2 * G + threadIdx.x];
  }
  load_q(f0.x);
  issue_next(A, false);                            // its K/V rows are already on the way
  if (staged) {                                    // visible after the first run's barrier
#pragma unroll
    for (int k = 0; k < Q2N; ++k) {
      const int t = threadIdx.x + k * AT_NT;
      if (t < G * D) s_q2[t / D][t % D] = q2v[k] * qscale;
    }
    if (threadIdx.x < G) s_m2[threadIdx.x] = (float)(m2v * (double)LOG2E);
  }
  reset();

  // one step: issue the next batch into `nxt`, reduce `cur`, close its run if it was
  // the run's last batch; false once the worker is done.  The two steps of the ring are
  // separate instances (the markers keep the compiler from folding them into one body,
  // which would reuse registers still being loaded and wait for them).
  auto step = [&](auto id, Batch &cur, Batch &nxt) -> bool {
    asm volatile("; pivot ring step %0" ::"n"(decltype(id)::value));
    if (!cur.live) return false;
    if (cur.first && cur.run > 0) {                // a new run: its queries, zero partials
      if (cur.run == 1 && staged)
        load_q_lds();
      else
        load_q(cur.unit);
      reset();
    }
    issue_next(nxt, true);
    __builtin_amdgcn_sched_barrier(0);             // keep the loads ahead of the reduction
    consume(cur);
    if (cur.last) epilogue(cur.slot);
    asm volatile("; pivot ring step end %0" ::"n"(decltype(id)::value));
    return true;
  };
  while (step(std::integral_constant<int, 0>{}, A, B) && step(std::integral_constant<int, 1>{}, B, A)) {
  }
}

template <bool BF16, int G>
static hipError_t launch_attend_g(const AttendArgs &a, int units, bool host, bool exact,
                                  hipStream_t st) {
  if (!host) {
    // persistent workers, as many as the schedule was made for (nsplit)
    return launch_kernel(k_attend_piv<BF16, G>, dim3(a.nsplit), dim3(AT_NT), 0, st, a);
  }
  if (exact) return launch_attend_t<BF16, G, true, true>(a, units, st);
  return launch_attend_t<BF16, G, true, false>(a, units, st);
}

hipError_t launch_attend(const AttendArgs &a, int units, bool bf16, bool host, bool exact,
                         hipStream_t st) {
  switch (a.t.G * 2 + (bf16 ? 1 : 0)) {
#define VERKV_AT_CASE(GG)                                                              \
  case GG * 2 + 1: return launch_attend_g<true, GG>(a, units, host, exact, st);        \
  case GG * 2: return launch_attend_g<false, GG>(a, units, host, exact, st);
    VERKV_AT_CASE(1) VERKV_AT_CASE(2) VERKV_AT_CASE(3) VERKV_AT_CASE(4)
    VERKV_AT_CASE(5) VERKV_AT_CASE(6) VERKV_AT_CASE(7) VERKV_AT_CASE(8)
#undef VERKV_AT_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace verkv
