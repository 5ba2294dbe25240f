// KVFetch steps 2-4 for gfx950, all in float64 ("Verify Before You Fetch", picx.dev
// summary page, "Methodology"):
//   * Definition 2: lambda_i = clip_[r_i,1](beta r_i / (w_i (1 - r_i))) with the bias
//     beta = sum_L w_i (1 - lambda_i) taken self-consistent.  beta is the unique root
//     of B = f(B), f piecewise linear and non-increasing; it is found by a safeguarded
//     Newton iteration that stops once the root of the current linear piece lies on
//     that piece (then it is exact).  kappa multiplies beta inside the clip.
//   * Lemma 1 / eq. (7): eps_hat(L) = E(beta, V, b) / D with
//     E = beta + b l/3 + sqrt((b l/3)^2 + 2 V l), l = log(2/delta), D = sum of all
//     sketch weights; certified iff eps_hat < eps.
//   * eqs. (9)-(10): g_i = eps_hat(L) - eps_hat(L \ {i}) with lambda frozen; the fetch
//     set is the k* tokens of largest g (ties: lower token index first) where k* is
//     the least k with eps_hat(L_g[k:]) < eps.
// The k* cut is found without sorting L: a most-significant-digit search over the
// bits of g (9-bit digits, then the token index for exact ties) keeps per-bucket
// counts, sums of beta_i and V_i and the maximum b_i in LDS, walks the buckets in
// ascending g to the first one whose inclusion pushes E(L') to eps*D, and recurses
// into it until at most WIN tokens remain.  Those are sorted in LDS (bitonic) and
// scanned against a deterministic re-sum of everything below them.  The tokens of F
// are OR-ed into the KV head's fetch bitmask (the union over the GQA group).
//
// Parallel layout: a query row is served by a team of T workgroups of 512 threads,
// each owning a contiguous slice of the row's tokens (T = 16 puts the 32 rows of a
// 32-query-head layer on all 256 CUs, two workgroups per CU).  Every reduction is first done inside the
// workgroup, then combined across the team in a fixed member order after a barrier
// on a counter in global memory; for the histograms every member sums all members'
// copies in member order.  Every member therefore sees identical
// combined values and takes the same path through the phases.  With T > 1 the grid
// never exceeds what the device holds at once, so whole teams are resident; a
// barrier wait is bounded and reports a timeout in the status word instead of
// hanging.  With T = 1 the barriers reduce to workgroup barriers and any grid works.
#include "decide_util.h"

#include <algorithm>
#include <atomic>

namespace verkv {

__global__ __launch_bounds__(DC_NT) void k_decide(DecideArgs a) {
  extern __shared__ double s_dyn[];          // [nch] chunk scales, then [4][LDS_TOK] cache
  __shared__ double scr[NQ * DC_NW];
  __shared__ double s_part[TEAM_MAX * PART];
  __shared__ uint32_t h_cnt[NBUCKET];
  __shared__ double h_beta[NBUCKET];
  __shared__ double h_V[NBUCKET];
  __shared__ uint64_t h_b[NBUCKET];
  __shared__ uint64_t w_key[WIN];
  __shared__ uint32_t w_lo[WIN];
  __shared__ int32_t s_int[4];

  const int T = a.team;
  int row, m;
  if (a.xcd_map) {                      // members of a team on the same XCD (round-robin dispatch)
    const int idx = blockIdx.x >> 3;
    row = (idx / T) * 8 + (blockIdx.x & 7);
    m = idx % T;
  } else {
    row = blockIdx.x / T;
    m = blockIdx.x % T;
  }
  {                                     // dispatch order: the longest sequences' rows first
    const int hq = a.t.Hkv * a.t.G;
    row = (int)a.t.order[row / hq] * hq + row % hq;
  }
  const int Hq = a.t.Hkv * a.t.G;
  const int b = row / Hq;
  const int h = row % Hq;
  const int g = h / a.t.G;
  const int n = a.t.s[b].n;
  const int nch = chunks_of(n);
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int s0 = (int)((int64_t)n * m / T);
  const int s1 = (int)((int64_t)n * (m + 1) / T);
  const bool cached = (s1 - s0) <= TR * DC_NT;        // selection terms in registers
  const bool lcache = (s1 - s0) <= LDS_TOK && a.lds_cache;  // (w, r, 1/r, r/(1-r)) in LDS
  double *s_scale = s_dyn;
  double *s_w = s_dyn + a.nch_max;
  double *s_r = s_w + LDS_TOK;
  double *s_ir = s_r + LDS_TOK;
  double *s_rq = s_ir + LDS_TOK;
  const double *wcr = a.wc + row_tok_base(a.t, b, h);
  const double2 *cs = a.cstat + row_chunk_base(a.t, b, h);
  const double *rr = a.r + tok_base(a.t, b, g);
  uint32_t *fb = a.fbits + word_base(a.t, b, g);
  const double kappa = a.kappa, l = a.l, eps = a.eps;
  // exchange slots of this row, member stride TW (the workspace's team size)
  const int TW = a.team_ws;
  double *xseq = a.xseq + (int64_t)row * 2 * TW;              // [2][TW] sequence words
  double *part = a.part + (int64_t)row * 2 * TW * PART;       // [2][TW][PART]
  uint32_t nx = 0;                                             // exchanges done
#define XPAR() ((int)((nx + 1) & 1))                            // parity of the next exchange
#define TEAM_SYNC()                                                         \
  do {                                                                      \
    if (T > 1) { ++nx; team_exchange(xseq + (nx & 1) * TW, m, T, nx, a.status); } \
    else __syncthreads();                                                   \
  } while (0)
#define SLOT() (part + (int64_t)XPAR() * TW * PART)
  // exchange: every member has stored its PART values into `sl` (tid 0); after the
  // exchange the team's partials are staged in LDS with one parallel load
#define TEAM_STAGE(sl)                                                      \
  do {                                                                      \
    TEAM_SYNC();                                                            \
    for (int j_ = tid; j_ < T * PART; j_ += DC_NT) s_part[j_] = xget((sl) + j_); \
    __syncthreads();                                                        \
  } while (0)
#ifdef VERKV_PHASE_TIMING
  int nstamp = 0;
#define STAMP()                                                                                  \
  do {                                                                                           \
    if (tid == 0 && a.phase_clock && nstamp < 32) {                                              \
      a.phase_clock[((int64_t)row * T + m) * 64 + nstamp] = wall_clock64();                      \
      a.phase_clock[((int64_t)row * T + m) * 64 + 32 + nstamp] = clock64();                      \
    }                                                                                            \
    ++nstamp;                                                                                    \
  } while (0)
#else
#define STAMP() do {} while (0)
#endif
  STAMP();

  // read before the first team exchange; member 0 overwrites it at the end
  const double bwarm = a.bprev ? a.bprev[row] : 0.0;

  // the slice's r and chunk-relative weights, loaded before the reductions below so
  // their latency overlaps them (kept only when the slice goes to the LDS cache)
  double rb0[TR], wb0[TR];
  if (lcache) {
#pragma unroll
    for (int k = 0; k < TR; ++k) {
      const int i = s0 + tid + k * DC_NT;
      rb0[k] = i < s1 ? rr[i] : 2.0;
      wb0[k] = i < s1 ? wcr[i] : 0.0;
    }
  }

  // ---- step 1 (finish): m_hat, per-chunk rescale, D (every member, same order)
  double mloc = -INFINITY;
  for (int c = tid; c < nch; c += DC_NT) mloc = fmax(mloc, cs[c].x);
  const double m_hat = block_max<DC_NT>(mloc, scr);
  double dloc = 0.0;
  for (int c = tid; c < nch; c += DC_NT) {
    const double sc = exp(cs[c].x - m_hat);
    s_scale[c] = sc;
    if (m == 0) a.cscale[row_chunk_base(a.t, b, h) + c] = sc;
    dloc += sc * cs[c].y;
  }
  const double Dd = block_sum<DC_NT>(dloc, scr);      // barrier also publishes s_scale
  const double *cz = a.cf0 + row_chunk_base(a.t, b, h);
  double zloc = 0.0;
  for (int c = tid; c < nch; c += DC_NT) zloc += s_scale[c] * cz[c];
  const double f0 = block_sum<DC_NT>(zloc, scr);      // f(0) = sum_L w (1 - r)

  // (w, r) of the slice in LDS, with 1/r and r/(1-r) for the fixed-point passes;
  // r >= 1 marks a token of H
  if (lcache) {
#pragma unroll
    for (int k = 0; k < TR; ++k) {
      const int i = s0 + tid + k * DC_NT;
      if (i >= s1) continue;
      const double ri = rb0[k];
      const bool inL = ri < 1.0;
      s_r[i - s0] = ri;
      s_w[i - s0] = inL ? wb0[k] * s_scale[i / SKETCH_CHUNK] : 0.0;
      s_ir[i - s0] = inL && ri > 0.0 ? 1.0 / ri : 0.0;
      s_rq[i - s0] = inL ? ri / (1.0 - ri) : 0.0;
    }
    __syncthreads();
  }
  STAMP();

#define FOR_L(body)                                                   \
  if (lcache) {                                                       \
    for (int i = s0 + tid; i < s1; i += DC_NT) {                      \
      const double ri = s_r[i - s0];                                  \
      if (!(ri < 1.0)) continue;                                      \
      const double wi = s_w[i - s0];                                  \
      body                                                            \
    }                                                                 \
  } else {                                                            \
    for (int i0 = s0 + tid; i0 < s1; i0 += SB * DC_NT) {              \
      double rb[SB], wb[SB];                                          \
      _Pragma("unroll")                                               \
      for (int u = 0; u < SB; ++u) {                                  \
        const int iu = i0 + u * DC_NT;                                \
        rb[u] = iu < s1 ? rr[iu] : 2.0;                               \
        wb[u] = iu < s1 ? wcr[iu] : 0.0;                              \
      }                                                               \
      _Pragma("unroll")                                               \
      for (int u = 0; u < SB; ++u) {                                  \
        const int i = i0 + u * DC_NT;                                 \
        const double ri = rb[u];                                      \
        if (!(ri < 1.0)) continue;                                    \
        const double wi = wb[u] * s_scale[i / SKETCH_CHUNK];          \
        body                                                          \
      }                                                               \
    }                                                                 \
  }

  // FOR_L with the reciprocals of r: ir = 1/r, rq = r/(1-r) (0 where r = 0)
#define FOR_LX(body)                                                  \
  if (lcache) {                                                       \
    for (int i0 = s0 + tid; i0 < s1; i0 += 4 * DC_NT) {               \
      double rb[4], wb[4], ib[4], qb[4];                              \
      _Pragma("unroll")                                               \
      for (int u = 0; u < 4; ++u) {                                   \
        const int iu = i0 + u * DC_NT;                                \
        const bool ok = iu < s1;                                      \
        rb[u] = ok ? s_r[iu - s0] : 2.0;                              \
        wb[u] = ok ? s_w[iu - s0] : 0.0;                              \
        ib[u] = ok ? s_ir[iu - s0] : 0.0;                             \
        qb[u] = ok ? s_rq[iu - s0] : 0.0;                             \
      }                                                               \
      _Pragma("unroll")                                               \
      for (int u = 0; u < 4; ++u) {                                   \
        const double ri = rb[u];                                      \
        if (!(ri < 1.0)) continue;                                    \
        const double wi = wb[u];                                      \
        const double ir = ib[u];                                      \
        const double rq = qb[u];                                      \
        body                                                          \
      }                                                               \
    }                                                                 \
  } else {                                                            \
    FOR_L(                                                            \
      const double ir = ri > 0.0 ? 1.0 / ri : 0.0;                    \
      const double rq = ri / (1.0 - ri);                              \
      body)                                                           \
  }

  auto combine_sum1 = [&](double v) -> double {
    if (T == 1) return v;
    double *sl = SLOT();
    if (tid == 0) xput(sl + m * PART, v);
    TEAM_STAGE(sl);
    double t = 0.0;
    for (int k = 0; k < T; ++k) t += s_part[k * PART];
    return t;
  };

  // ---- self-consistent beta (Definition 2) and the eq. (7) totals
  double Bst = 0.0;
  Cert ct{0.0, 0.0, 0.0, 0.0};
  double nLt = 0.0;
  bool have_cert = false;
  if (isinf(kappa) || kappa == 0.0) {
    double acc = 0.0;
    if (isinf(kappa)) { FOR_L(if (ri == 0.0) acc += wi;) }
    else { FOR_L(acc += wi * (1.0 - ri);) }
    Bst = combine_sum1(block_sum<DC_NT>(acc, scr));
  } else if (f0 > 0.0) {
    // safeguarded Newton inside the bracket [0, f(0)], from this row's B* of the last
    // step when the workspace holds one in the bracket (the result is the root of the
    // final linear piece, whatever the start), else from f(0)
    double lo = 0.0, hi = f0, B = (bwarm > 0.0 && bwarm < f0) ? bwarm : f0;
    const double inv_kappa = 1.0 / kappa;
    bool done = false;
    for (int iter = 0; iter < 200; ++iter) {
      NewtonAcc v{0.0, 0.0, 0.0, INFINITY, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
      // per token: lambda = r below aa = w (1 - r) / kappa, 1 above tt = aa / r, linear
      // in between; with 1/r and r/(1-r) at hand every term is a product
      FOR_LX(newton_add(v, ri, wi, ir, rq, B, kappa, inv_kappa);)
      STAMP();
      // the step needs only the linear model and its piece; the eq. (7) totals of the
      // pass are reduced once the root is found to lie on that piece
      Lin lm = block_lin(v, scr);
      STAMP();
      if (T > 1) {
        double *sl = SLOT();
        if (tid == 0) {
          double *q = sl + m * PART;
          xput(q + 0, lm.c0); xput(q + 1, lm.c1); xput(q + 2, lm.lo); xput(q + 3, lm.hi);
        }
        TEAM_STAGE(sl);
        lm = Lin{0.0, 0.0, 0.0, INFINITY};
        for (int k = 0; k < T; ++k) {
          const double *q = s_part + k * PART;
          lm.c0 += q[0]; lm.c1 += q[1]; lm.lo = fmax(lm.lo, q[2]); lm.hi = fmin(lm.hi, q[3]);
        }
      }
      STAMP();
      const double hB = B * (1.0 + lm.c1) - lm.c0;       // B - f(B)
      const double Bn = lm.c0 / (1.0 + lm.c1);           // root of this linear piece
      Bst = Bn;
      bool on_piece = (Bn >= lm.lo && Bn <= lm.hi);
      if (!on_piece && hB == 0.0) { Bst = B; on_piece = true; }
      if (on_piece) {
        NewtonAcc o = block_newton(v, scr);
        if (T > 1) {
          double *sl = SLOT();
          if (tid == 0) {
            double *q = sl + m * PART;
            xput(q + 4, o.vc); xput(q + 5, o.vm); xput(q + 6, o.cnt); xput(q + 7, o.bc1);
            xput(q + 8, o.bc2); xput(q + 9, o.bm1); xput(q + 10, o.bm2);
          }
          TEAM_STAGE(sl);
          o = NewtonAcc{lm.c0, lm.c1, lm.lo, lm.hi, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
          for (int k = 0; k < T; ++k) {
            const double *q = s_part + k * PART;
            o.vc += q[4]; o.vm += q[5]; o.cnt += q[6];
            top2_merge(o.bc1, o.bc2, q[7], q[8]);
            top2_merge(o.bm1, o.bm2, q[9], q[10]);
          }
        }
        // the totals of eq. (7) on this piece, at B = Bst
        ct.beta = o.c0 - Bst * o.c1;
        ct.V = o.vc + Bst * Bst * o.vm;
        ct.b1 = o.bc1; ct.b2 = o.bc2;
        top2_merge(ct.b1, ct.b2, Bst * o.bm1, Bst * o.bm2);
        nLt = o.cnt;
        have_cert = true;
        done = true;
        break;
      }
      if (hB < 0.0) lo = B; else hi = B;
      double Bnext = Bn;
      if (!(Bnext > lo && Bnext < hi)) Bnext = 0.5 * (lo + hi);
      if (Bnext == B || !(hi > lo)) { done = true; break; }
      B = Bnext;
    }
    if (!done && tid == 0 && m == 0) atomicOr(a.status, 2);
  }

  // per-token terms at B*: one formula for every pass of this kernel (tokens of this
  // member's slice take 1/r and r/(1-r) from the LDS cache, others compute them the
  // same way)
  const double kB = kappa * Bst;
  const bool kinf = isinf(kappa);
  auto tok_terms = [&](int i, double wi, double ri, bool local) -> Terms {
    double ir, rq;
    if (local && lcache) { ir = s_ir[i - s0]; rq = s_rq[i - s0]; }
    else { ir = ri > 0.0 ? 1.0 / ri : 0.0; rq = ri / (1.0 - ri); }
    return terms_at(wi, ri, ir, rq, kB, kinf);
  };

  if (!have_cert) {
    Cert cl{0.0, 0.0, 0.0, 0.0};
    int nL = 0;
    FOR_L(
      const Terms x = tok_terms(i, wi, ri, true);
      cl.beta += x.beta; cl.V += x.V; ++nL;
      top2_merge(cl.b1, cl.b2, x.b, 0.0);)
    ct = block_cert(cl, scr);
    nLt = block_sum<DC_NT>((double)nL, scr);
    if (T > 1) {
      double *sl = SLOT();
      if (tid == 0) {
        double *q = sl + m * PART;
        xput(q + 0, ct.beta); xput(q + 1, ct.V); xput(q + 2, ct.b1); xput(q + 3, ct.b2); xput(q + 4, nLt);
      }
      TEAM_STAGE(sl);
      ct = Cert{0.0, 0.0, 0.0, 0.0};
      nLt = 0.0;
      for (int k = 0; k < T; ++k) {
        const double *q = s_part + k * PART;
        ct = cert_combine(ct, Cert{q[0], q[1], q[2], q[3]});
        nLt += q[4];
      }
    }
  }
  STAMP();
  const double E_all = nLt > 0.0 ? bern_E(ct.beta, ct.V, ct.b1, l) : 0.0;
  const double ehat = E_all / Dd;
  const bool cert = ehat < eps;
  if (tid == 0 && m == 0) {
    if (row == 0) { a.params[0] = kappa; a.params[1] = l; }
    a.m_hat[row] = m_hat;
    a.d_sketch[row] = Dd;
    a.beta_star[row] = Bst;
    if (a.bprev) a.bprev[row] = Bst;
    a.eps_hat[row] = ehat;
    a.certified[row] = cert ? 1 : 0;
  }
  if (cert) return;                                    // kstar was cleared before the kernel
  const double t1x = ct.b1 * l / 3.0;
  const double sqX = sqrt(t1x * t1x + 2.0 * ct.V * l);   // sqrt(X) of g_of, once per row
  if (a.resolved) {
    // the cut with the bias re-solved per candidate set is made by k_resolve, from the
    // same fetch keys: hand it the totals of the full L they are formed with
    if (tid == 0 && m == 0) {
      a.gpar[4 * row] = ct.V; a.gpar[4 * row + 1] = ct.b1;
      a.gpar[4 * row + 2] = ct.b2; a.gpar[4 * row + 3] = sqX;
    }
    return;
  }

  // ---- eqs. (9)-(10): MSD search for the k* cut over the bits of g
  // per-token terms and keys, cached for the remaining passes
  uint64_t ckey[TR];
  double cbeta[TR], cV[TR], cb[TR];
  bool cin[TR];
#pragma unroll
  for (int k = 0; k < TR; ++k) {
    ckey[k] = 0; cbeta[k] = 0.0; cV[k] = 0.0; cb[k] = 0.0; cin[k] = false;
    const int i = s0 + tid + k * DC_NT;
    if (cached && i < s1) {
      const double ri = lcache ? s_r[i - s0] : rr[i];
      if (ri < 1.0) {
        const double wi = lcache ? s_w[i - s0] : wcr[i] * s_scale[i / SKETCH_CHUNK];
        const Terms x = tok_terms(i, wi, ri, true);
        cbeta[k] = x.beta; cV[k] = x.V; cb[k] = x.b;
        ckey[k] = dbits(g_of(x, ct.V, ct.b1, ct.b2, l, Dd, sqX));
        cin[k] = true;
      }
    }
  }
#define FOR_SEL(body)                                                          \
  if (cached) {                                                                \
    _Pragma("unroll")                                                          \
    for (int k = 0; k < TR; ++k) {                                             \
      if (!cin[k]) continue;                                                   \
      const int i = s0 + tid + k * DC_NT;                                      \
      const uint64_t key = ckey[k];                                            \
      const uint32_t lo = IDX_MAX - (uint32_t)i;                               \
      const Terms x{cbeta[k], cV[k], cb[k]};                                   \
      body                                                                     \
    }                                                                          \
  } else {                                                                     \
    for (int i = s0 + tid; i < s1; i += DC_NT) {                               \
      const double ri = rr[i];                                                 \
      if (!(ri < 1.0)) continue;                                               \
      const double wi = wcr[i] * s_scale[i / SKETCH_CHUNK];                    \
      const Terms x = tok_terms(i, wi, ri, true);                              \
      const uint64_t key = dbits(g_of(x, ct.V, ct.b1, ct.b2, l, Dd, sqX));     \
      const uint32_t lo = IDX_MAX - (uint32_t)i;                               \
      body                                                                     \
    }                                                                          \
  }

  STAMP();
  const double thr = eps * Dd;
  double bel_beta = 0.0, bel_V = 0.0, bel_b = 0.0;     // tokens below the window
  uint64_t pkey = 0;
  uint32_t plo = 0;
  int lev = -1;
  bool above_mode = false;                               // cut above the whole window
  const int64_t hrow = (int64_t)row * 2 * TW * NBUCKET;       // [2][TW][NBUCKET] per row

  for (int L = 0; L < NLEV; ++L) {
    for (int k = tid; k < NBUCKET; k += DC_NT) { h_cnt[k] = 0; h_beta[k] = 0.0; h_V[k] = 0.0; h_b[k] = 0; }
    __syncthreads();
    const int sh = c_lev_shift[L];
    const uint32_t dmask = (1u << c_lev_width[L]) - 1u;
    auto hist_tok = [&](bool act, uint64_t key, uint32_t lo, const Terms &x) {
      const uint32_t dig = c_lev_lo[L] ? ((lo >> sh) & dmask) : (uint32_t)((key >> sh) & dmask);
      if (act) {
        atomicAdd(&h_cnt[dig], 1u);
        atomicAdd(&h_beta[dig], x.beta);
        atomicAdd(&h_V[dig], x.V);
        atomicMax((unsigned long long *)&h_b[dig], (unsigned long long)dbits(x.b));
      }
    };
    if (cached) {
      // A thread first merges its own TR tokens that share a bucket (the first digit
      // holds exponent bits of g, so a few buckets take most tokens and the LDS
      // atomics on them serialise); then one update per distinct bucket.
      uint32_t dg[TR], cn[TR];
      double sbeta[TR], sV[TR], smb[TR];
#pragma unroll
      for (int k = 0; k < TR; ++k) {
        const int i = s0 + tid + k * DC_NT;
        const uint32_t lo = IDX_MAX - (uint32_t)i;
        const bool act = cin[k] && cmp_window(ckey[k], lo, lev, pkey, plo) == 0;
        dg[k] = c_lev_lo[L] ? ((lo >> sh) & dmask) : (uint32_t)((ckey[k] >> sh) & dmask);
        cn[k] = act ? 1u : 0u;
        sbeta[k] = act ? cbeta[k] : 0.0;
        sV[k] = act ? cV[k] : 0.0;
        smb[k] = act ? cb[k] : 0.0;
      }
#pragma unroll
      for (int k = 1; k < TR; ++k) {
#pragma unroll
        for (int j = 0; j < k; ++j) {
          if (cn[k] && cn[j] && dg[j] == dg[k]) {
            cn[j] += cn[k]; sbeta[j] += sbeta[k]; sV[j] += sV[k]; smb[j] = fmax(smb[j], smb[k]);
            cn[k] = 0;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < TR; ++k) {
        if (cn[k]) {
          atomicAdd(&h_cnt[dg[k]], cn[k]);
          atomicAdd(&h_beta[dg[k]], sbeta[k]);
          atomicAdd(&h_V[dg[k]], sV[k]);
          atomicMax((unsigned long long *)&h_b[dg[k]], (unsigned long long)dbits(smb[k]));
        }
      }
    } else {
      for (int i0 = s0; i0 < s1; i0 += DC_NT) {
        const int i = i0 + tid;
        const uint32_t lo = IDX_MAX - (uint32_t)i;
        bool act = false;
        uint64_t key = 0;
        Terms x{0.0, 0.0, 0.0};
        if (i < s1) {
          const double ri = rr[i];
          if (ri < 1.0) {
            const double wi = wcr[i] * s_scale[i / SKETCH_CHUNK];
            x = tok_terms(i, wi, ri, true);
            key = dbits(g_of(x, ct.V, ct.b1, ct.b2, l, Dd, sqX));
            act = cmp_window(key, lo, lev, pkey, plo) == 0;
          }
        }
        hist_tok(act, key, lo, x);
      }
    }
    __syncthreads();
    STAMP();
    if (T > 1) {
      // publish this member's histogram; after the barrier every member sums all of
      // them in member order, so all hold the same merged histogram
      const int64_t hp = hrow + (int64_t)XPAR() * TW * NBUCKET;   // this exchange's buffer
      const int64_t hm = hp + (int64_t)m * NBUCKET;
      for (int k = tid; k < NBUCKET; k += DC_NT) {
        xput(a.hcnt + hm + k, h_cnt[k]); xput(a.hbeta + hm + k, h_beta[k]);
        xput(a.hV + hm + k, h_V[k]); xput(a.hmax + hm + k, h_b[k]);
      }
      TEAM_SYNC();
      STAMP();
      for (int k = tid; k < NBUCKET; k += DC_NT) {
        uint32_t c = 0; double sb = 0.0, sv = 0.0; uint64_t mb = 0;
        for (int q0 = 0; q0 < T; q0 += 4) {          // four members' loads in flight
          uint32_t qc[4]; double qb[4], qv[4]; uint64_t qm[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            qc[u] = 0; qb[u] = 0.0; qv[u] = 0.0; qm[u] = 0;
            if (q0 + u < T) {
              const int64_t o = hp + (int64_t)(q0 + u) * NBUCKET + k;
              qc[u] = xget(a.hcnt + o); qb[u] = xget(a.hbeta + o); qv[u] = xget(a.hV + o); qm[u] = xget(a.hmax + o);
            }
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (q0 + u < T) { c += qc[u]; sb += qb[u]; sv += qv[u]; mb = qm[u] > mb ? qm[u] : mb; }
          }
        }
        h_cnt[k] = c; h_beta[k] = sb; h_V[k] = sv; h_b[k] = mb;
      }
      __syncthreads();
      STAMP();
    }
    // inclusive scan over buckets (thread k owns bucket k): beta, V sums and max b
    double sb = h_beta[tid], sv = h_V[tid], smx = bitsd(h_b[tid]);
    const uint32_t mycnt = h_cnt[tid];
    __syncthreads();
    for (int off = 1; off < NBUCKET; off <<= 1) {
      double ob = 0.0, ov = 0.0, om = 0.0;
      if (tid >= off) { ob = h_beta[tid - off]; ov = h_V[tid - off]; om = bitsd(h_b[tid - off]); }
      __syncthreads();
      if (tid >= off) { sb += ob; sv += ov; smx = fmax(smx, om); }
      h_beta[tid] = sb; h_V[tid] = sv; h_b[tid] = dbits(smx);
      __syncthreads();
    }
    if (tid == 0) s_int[0] = INT32_MAX;
    __syncthreads();
    const bool below_fails = bern_E(bel_beta, bel_V, bel_b, l) >= thr;
    if (mycnt > 0 &&
        (below_fails || bern_E(bel_beta + sb, bel_V + sv, fmax(bel_b, smx), l) >= thr))
      atomicMin(&s_int[0], tid);
    __syncthreads();
    const int j = s_int[0];
    if (j == INT32_MAX) { above_mode = true; break; }
    const double eb = j > 0 ? h_beta[j - 1] : 0.0;
    const double ev = j > 0 ? h_V[j - 1] : 0.0;
    const double em = j > 0 ? bitsd(h_b[j - 1]) : 0.0;
    bel_beta += eb; bel_V += ev; bel_b = fmax(bel_b, em);
    if (!c_lev_lo[L]) {
      pkey = (L == 0) ? (uint64_t)j : ((pkey << c_lev_width[L]) | (uint64_t)j);
    } else {
      plo = (L == FIRST_LO_LEV) ? (uint32_t)j : ((plo << c_lev_width[L]) | (uint32_t)j);
    }
    lev = L;
    const uint32_t cntj = h_cnt[j];
    __syncthreads();
    STAMP();
    if (cntj <= (uint32_t)WIN) break;
  }

  // ---- final window: deterministic re-sum below it, sort it, scan it
  uint64_t tkey = 0;
  uint32_t tlo = 0;
  if (!above_mode) {
    if (tid == 0) s_int[1] = 0;
    for (int k = tid; k < WIN; k += DC_NT) { w_key[k] = ~0ull; w_lo[k] = ~0u; }
    __syncthreads();
    uint64_t *gkey = a.wkey + (int64_t)row * WIN;
    uint32_t *glo = a.wlo + (int64_t)row * WIN;
    Red4 bel{0.0, 0.0, 0.0, 0.0};
    FOR_SEL(
      const int cw2 = cmp_window(key, lo, lev, pkey, plo);
      if (cw2 < 0) { bel.s0 += x.beta; bel.s1 += x.V; bel.mx = fmax(bel.mx, x.b); }
      else if (cw2 == 0) {
        if (T > 1) {
          const uint32_t p = atomicAdd(&a.wcount[row], 1u);
          if (p < (uint32_t)WIN) { xput(gkey + p, key); xput(glo + p, lo); }
        } else {
          const int p = atomicAdd(&s_int[1], 1);
          if (p < WIN) { w_key[p] = key; w_lo[p] = lo; }
        }
      })
    STAMP();
    Red4 bo = block_red4(bel, scr);
    int wcount;
    if (T > 1) {
      double *sl = SLOT();
      if (tid == 0) { xput(sl + m * PART, bo.s0); xput(sl + m * PART + 1, bo.s1); xput(sl + m * PART + 2, bo.mx); }
      TEAM_STAGE(sl);
      bo = Red4{0.0, 0.0, 0.0, 0.0};
      for (int k = 0; k < T; ++k) {
        bo.s0 += s_part[k * PART]; bo.s1 += s_part[k * PART + 1]; bo.mx = fmax(bo.mx, s_part[k * PART + 2]);
      }
      wcount = min((int)__hip_atomic_load(&a.wcount[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), WIN);
      for (int k = tid; k < wcount; k += DC_NT) { w_key[k] = xget(gkey + k); w_lo[k] = xget(glo + k); }
      __syncthreads();
    } else {
      wcount = min(s_int[1], WIN);
    }
    STAMP();
    const bool bfail = bern_E(bo.s0, bo.s1, bo.mx, l) >= thr;
    if (tid == 0) s_int[2] = INT32_MAX;
    __syncthreads();
    if (wcount <= WAVE) {
      // one wave sorts and scans the window in registers
      if (tid < WAVE) {
        uint64_t key = lane < wcount ? w_key[lane] : ~0ull;
        uint32_t lo = lane < wcount ? w_lo[lane] : ~0u;
        wave_bitonic(key, lo);
        double tb = 0.0, tv = 0.0, tm = 0.0;
        if (lane < wcount) {
          const int i = (int)(IDX_MAX - lo);
          const double ri = rr[i];
          const double wi = wcr[i] * s_scale[i / SKETCH_CHUNK];
          const Terms x = tok_terms(i, wi, ri, false);
          tb = x.beta; tv = x.V; tm = x.b;
        }
        for (int off = 1; off < WAVE; off <<= 1) {
          const double ob = __shfl_up(tb, off, WAVE), ov = __shfl_up(tv, off, WAVE),
                       om = __shfl_up(tm, off, WAVE);
          if (lane >= off) { tb += ob; tv += ov; tm = fmax(tm, om); }
        }
        const bool fails = lane < wcount &&
                           (bfail || bern_E(bo.s0 + tb, bo.s1 + tv, fmax(bo.mx, tm), l) >= thr);
        const uint64_t fm = __ballot(fails);
        const int jc = fm ? __ffsll((long long)fm) - 1 : 0;      // uniform in the wave
        const uint64_t kj = __shfl(key, jc, WAVE);                // whole wave active
        const uint32_t lj = __shfl(lo, jc, WAVE);
        if (lane == 0 && fm) {
          s_int[2] = jc;
          w_key[0] = kj;
          w_lo[0] = lj;
        }
      }
      __syncthreads();
      if (s_int[2] == INT32_MAX) above_mode = true;
      else { tkey = w_key[0]; tlo = w_lo[0]; }
    } else {
      // bitonic sort of (key, lo) ascending over the next power of two >= wcount
      int P = 128;
      while (P < wcount) P <<= 1;     // wcount <= WIN == DC_NT
      for (int k2 = 2; k2 <= P; k2 <<= 1) {
        for (int j2 = k2 >> 1; j2 > 0; j2 >>= 1) {
          const int p = tid ^ j2;
          if (tid < P && p > tid) {
            const uint64_t ka = w_key[tid], kb = w_key[p];
            const uint32_t la = w_lo[tid], lb = w_lo[p];
            const bool gt = (ka > kb) || (ka == kb && la > lb);
            const bool up = (tid & k2) == 0;
            if (gt == up) {
              w_key[tid] = kb; w_key[p] = ka;
              w_lo[tid] = lb; w_lo[p] = la;
            }
          }
          __syncthreads();
        }
      }
      double tb = 0.0, tv = 0.0, tm = 0.0;
      if (tid < wcount) {
        const int i = (int)(IDX_MAX - w_lo[tid]);
        const double ri = rr[i];
        const double wi = wcr[i] * s_scale[i / SKETCH_CHUNK];
        const Terms x = tok_terms(i, wi, ri, false);
        tb = x.beta; tv = x.V; tm = x.b;
      }
      h_beta[tid] = tb; h_V[tid] = tv; h_b[tid] = dbits(tm);
      __syncthreads();
      for (int off = 1; off < P; off <<= 1) {
        double ob = 0.0, ov = 0.0, om = 0.0;
        if (tid >= off) { ob = h_beta[tid - off]; ov = h_V[tid - off]; om = bitsd(h_b[tid - off]); }
        __syncthreads();
        if (tid >= off) { tb += ob; tv += ov; tm = fmax(tm, om); }
        h_beta[tid] = tb; h_V[tid] = tv; h_b[tid] = dbits(tm);
        __syncthreads();
      }
      if (tid < wcount && (bfail || bern_E(bo.s0 + tb, bo.s1 + tv, fmax(bo.mx, tm), l) >= thr))
        atomicMin(&s_int[2], tid);
      __syncthreads();
      const int jc = s_int[2];
      if (jc == INT32_MAX) above_mode = true;
      else { tkey = w_key[jc]; tlo = w_lo[jc]; }
    }
    __syncthreads();
  }

  STAMP();
  // ---- mark F_h = tokens at or after the cut in g-descending order
  // one ballot per wave and token group; at most three word ORs per wave instead of
  // one atomic per fetched token
  int64_t kc = 0;
  auto in_F = [&](uint64_t key, uint32_t lo) -> bool {
    if (above_mode) return cmp_window(key, lo, lev, pkey, plo) > 0;
    return (key > tkey) || (key == tkey && lo >= tlo);
  };
  if (cached) {
#pragma unroll
    for (int k = 0; k < TR; ++k) {
      const int i = s0 + tid + k * DC_NT;
      const bool f = cin[k] && in_F(ckey[k], IDX_MAX - (uint32_t)i);
      kc += f ? 1 : 0;
      or_bits_wave(fb, i - lane, f, lane);
    }
  } else {
    for (int i0 = s0; i0 < s1; i0 += DC_NT) {
      const int i = i0 + tid;
      bool f = false;
      if (i < s1) {
        const double ri = rr[i];
        if (ri < 1.0) {
          const double wi = wcr[i] * s_scale[i / SKETCH_CHUNK];
          const Terms x = tok_terms(i, wi, ri, true);
          f = in_F(dbits(g_of(x, ct.V, ct.b1, ct.b2, l, Dd, sqX)), IDX_MAX - (uint32_t)i);
        }
      }
      kc += f ? 1 : 0;
      or_bits_wave(fb, i - lane, f, lane);
    }
  }
  const int64_t ks = block_sum_i64<DC_NT>(kc, (int64_t *)scr);
  if (tid == 0 && ks) atomicAdd(&a.kstar[row], (int32_t)ks);
  STAMP();
#undef STAMP
#undef FOR_SEL
#undef FOR_LX
#undef FOR_L
#undef TEAM_STAGE
#undef TEAM_SYNC
#undef SLOT
}

// ------------------------------------------------------------------ fetch lists
// LS_NB blocks per KV head, each owning a contiguous run of 64-token groups (two
// bitmask words).  A block first counts the tokens of all groups before its run (a
// re-read of at most the head's whole bitmask), so no second launch is needed for the
// prefix.  Inside the block every wave owns a sub-run: pass 1 counts, a block scan
// gives each wave its first list position, pass 2 walks the groups in order, one lane
// per token, and writes the set bits with a ballot prefix so that consecutive list
// entries come from consecutive lanes (whole-line stores).  Lists are ascending.  A
// host-row entry also carries the token's staging slot + 1 above tok_bits (0 when the
// token is not staged); the host-row kernel checks the slot's token before using it.
constexpr int LS_NT = 256;
constexpr int LS_NB = 32;

__global__ __launch_bounds__(LS_NT) void k_lists(UnionArgs a) {
  __shared__ int32_t iscr[LS_NT / WAVE];
  constexpr int NWV = LS_NT / WAVE;
  const int unit = blockIdx.y;
  const int b = unit / a.t.Hkv;
  const int g = unit % a.t.Hkv;
  const int n = a.t.s[b].n;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wv = tid / WAVE;
  const uint32_t *fb = a.fbits + word_base(a.t, b, g);
  const uint32_t *res = a.resident + word_base(a.t, b, g);
  const int W = words_of(n);
  const int ngrp = (W + 1) / 2;
  const int per = (ngrp + LS_NB - 1) / LS_NB;
  const int B0 = min(ngrp, (int)blockIdx.x * per), B1 = min(ngrp, B0 + per);
  auto group_bits = [&](const uint32_t *wd, int gi) -> uint64_t {
    const uint64_t lo32 = wd[2 * gi];
    const uint64_t hi32 = 2 * gi + 1 < W ? wd[2 * gi + 1] : 0u;
    return lo32 | (hi32 << 32);
  };
  // the staging copies of this step have finished (they run before this kernel); when
  // they ran for this cache, entries are tagged with their slots and the header names
  // this cache as the one whose rows the maps hold
  const bool staged = a.shdr && a.shdr[6] == 1ull;
  if (a.stg_cnt && blockIdx.x == 0 && tid == 0) a.stg_cnt[unit] = 0;   // this step's count
  if (staged && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
    a.shdr[1] = a.ident_ptr;
    a.shdr[2] = a.ident_shape;
    a.shdr[0] = STAGE_MAGIC;
  }
  // the staging slot of each token of this head (-1: not staged), or none
  const int32_t *smap = (staged && a.slot_of) ? a.slot_of + tok_base(a.t, b, g) : nullptr;
  // tokens of F and of F \ S before this block's run
  int32_t cf = 0, ch = 0;
  for (int gi = tid; gi < B0; gi += LS_NT) {
    const uint64_t f = group_bits(fb, gi), r = group_bits(res, gi);
    cf += __popcll(f);
    ch += __popcll(f & ~r);
  }
  int32_t bf, bh;
  (void)block_excl_scan<LS_NT>(cf, iscr, &bf);
  (void)block_excl_scan<LS_NT>(ch, iscr, &bh);
  // this block's run, split over its waves
  const int gpw = (B1 - B0 + NWV - 1) / NWV;
  const int ga = min(B1, B0 + wv * gpw), gb = min(B1, ga + gpw);
  cf = 0;
  ch = 0;
  for (int gi = ga + lane; gi < gb; gi += WAVE) {
    const uint64_t f = group_bits(fb, gi), r = group_bits(res, gi);
    cf += __popcll(f);
    ch += __popcll(f & ~r);
  }
  cf = (int32_t)wave_sum_i64(cf);
  ch = (int32_t)wave_sum_i64(ch);
  int32_t tf, th;
  int32_t pf = block_excl_scan<LS_NT>(lane == 0 ? cf : 0, iscr, &tf);
  int32_t ph = block_excl_scan<LS_NT>(lane == 0 ? ch : 0, iscr, &th);
  pf = bf + __shfl(pf, 0, WAVE);            // the wave's first positions (lane 0's)
  ph = bh + __shfl(ph, 0, WAVE);
  int32_t *fl = a.fetch_idx ? a.fetch_idx + (int64_t)unit * a.fetch_cap : nullptr;
  int32_t *hl = a.h2d_idx + tok_base(a.t, b, g);
  const uint64_t below = (1ull << lane) - 1ull;
  // the slot of this lane's token in group gi (-1 past n or without staging)
  auto slot_at = [&](int gi) -> int32_t {
    const int tok = 64 * gi + lane;
    return (smap && gi < gb && tok < n) ? smap[tok] : -1;
  };
  for (int c0 = ga; c0 < gb; c0 += WAVE) {
    // lane j holds group c0 + j; the walk below takes them in order by shuffle
    uint64_t fl_l = 0, rl_l = 0;
    if (c0 + lane < gb) {
      fl_l = group_bits(fb, c0 + lane);
      rl_l = group_bits(res, c0 + lane);
    }
    const int nj = min(WAVE, gb - c0);
    int32_t sl_next = slot_at(c0);          // one group ahead of the walk
    for (int jj = 0; jj < nj; ++jj) {
      const uint64_t f = __shfl(fl_l, jj, WAVE), r = __shfl(rl_l, jj, WAVE);
      const int32_t sl = sl_next;
      sl_next = slot_at(c0 + jj + 1);
      const uint64_t hsel = f & ~r;
      const bool inf = (f >> lane) & 1ull, inh = (hsel >> lane) & 1ull;
      const int tok = 64 * (c0 + jj) + lane;
      if (inf) {
        const int32_t pos = pf + (int32_t)__popcll(f & below);
        if (fl && pos < a.fetch_cap) fl[pos] = tok;
      }
      if (inh) {
        // host-row entry: the token, and its staging slot + 1 when it is staged
        const uint32_t slot1 = (sl >= 0 && sl < a.stage_rows) ? (uint32_t)sl + 1u : 0u;
        hl[ph + (int32_t)__popcll(hsel & below)] = (int32_t)((uint32_t)tok | (slot1 << a.t.tok_bits));
      }
      pf += (int32_t)__popcll(f);
      ph += (int32_t)__popcll(hsel);
    }
  }
  if (blockIdx.x == LS_NB - 1 && tid == 0) {
    a.fetch_count[unit] = bf + tf;
    a.h2d_count[unit] = bh + th;
    if (a.h2d_count_ws) a.h2d_count_ws[unit] = bh + th;
  }
}

// ------------------------------------------------------------------ pivot coefficients
// Every resident pivot gets its estimator coefficient for every query row of the
// group: 1 on H and on S n F, lambda_i / r_i on S \ F (Definition 2 with the fetched
// tokens exact).
constexpr int UN_NT = 256;              // small blocks: they fit beside the host-row kernel

// The work schedule of the pivot attention, computed by one workgroup (a scan over the
// heads, then one thread per worker).  The pivots of
// KV head u fall into nc_u = ceil(cnt_u / PIVOT_CHUNK) chunks; the chunks of all heads,
// head after head, form one sequence of NC chunks, and worker w of P = min(workers, NC)
// takes chunks [floor(w NC / P), floor((w + 1) NC / P)): every worker gets the same
// number of rows to within a chunk, however ragged the heads are.  A worker sums its
// chunks of one head into one partial (a run); the runs of head u take the partial
// slots S_u .. S_u + runs_u - 1 in row order, S_u being the runs of the heads before u;
// runs[u] = {S_u, runs_u, C_u (the head's first chunk), 0}.
// Worker w's entry is a pair: {head, first row, end row, slot} of its first run, then
// {head, end row, slot, chunks left after it} of the second run when that is the next
// head's (head -1 otherwise, with the chunks left after the first run); {NC, P}
// follows the last pair.
__device__ void pivot_schedule(const PlanArgs &a) {
  __shared__ int32_t s_scan[UN_NT / WAVE];
  __shared__ int64_t s_sum[UN_NT / WAVE];
  const int units = a.t.B * a.t.Hkv;
  auto nc_of = [&](int u) -> int {
    const int c = min(max(a.piv_count[u], 0), a.cap);
    return (c + PIVOT_CHUNK - 1) / PIVOT_CHUNK;
  };
  int64_t mine = 0;
  for (int u = threadIdx.x; u < units; u += UN_NT) mine += nc_of(u);
  const int64_t NC = block_sum_i64<UN_NT>(mine, s_sum);
  const int64_t P = min((int64_t)a.workers, NC);
  for (int w = (int)P + threadIdx.x; w < a.workers; w += UN_NT) {
    a.sched[2 * w] = make_int4(0, 0, 0, 0);
    a.sched[2 * w + 1] = make_int4(0, 0, 0, 0);
  }
  if (threadIdx.x == 0) a.sched[2 * a.workers] = make_int4((int)NC, (int)P, 0, 0);
  // per head, tile by tile: C_u, runs_u and S_u (runs[u])
  int64_t carry = 0, slot_carry = 0;
  for (int t0 = 0; t0 < units; t0 += UN_NT) {
    const int u = t0 + threadIdx.x;
    const int ncu = u < units ? nc_of(u) : 0;
    int32_t tile = 0;
    const int64_t Cu = carry + block_excl_scan<UN_NT>(ncu, s_scan, &tile);
    carry += tile;
    // workers whose first chunk lies in [Cu, Cu + nc_u); run 0 belongs to an earlier
    // worker unless one of them starts exactly at Cu
    int runs = 0;
    if (ncu > 0) {
      const int64_t wlo = (Cu * P + NC - 1) / NC;
      const int64_t whi = ((Cu + ncu) * P + NC - 1) / NC;
      const int extra = (wlo < whi && wlo * NC / P == Cu) ? 0 : 1;
      runs = (int)(whi - wlo) + extra;
    }
    int32_t tile_runs = 0;
    const int64_t Su = slot_carry + block_excl_scan<UN_NT>(runs, s_scan, &tile_runs);
    slot_carry += tile_runs;
    if (u < units) a.runs[u] = make_int4((int)Su, runs, (int)Cu, 0);
  }
  __threadfence_block();
  __syncthreads();
  // per worker: its first chunk's head (the last head with C_u <= c0; a head without
  // chunks shares C_u with the next one), then the same entries as that head's loop
  for (int64_t w = threadIdx.x; w < P; w += UN_NT) {
    const int64_t c0 = w * NC / P, c1 = (w + 1) * NC / P;
    int lo = 0, hi = units - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)a.runs[mid].z <= c0) lo = mid; else hi = mid - 1;
    }
    const int u = lo;
    const int4 ru = a.runs[u];
    const int64_t Cu = ru.z;
    const int ncu = nc_of(u);
    const int64_t wlo = (Cu * P + NC - 1) / NC;
    const int extra = (wlo * NC / P == Cu) ? 0 : 1;
    const int cnt = min(max(a.piv_count[u], 0), a.cap);
    const int k0 = (int)(c0 - Cu);
    const int take = (int)min((int64_t)(ncu - k0), c1 - c0);
    const int p0 = k0 * PIVOT_CHUNK;
    const int left = (int)(c1 - c0) - take;
    a.sched[2 * w] = make_int4(u, p0, min(cnt, p0 + take * PIVOT_CHUNK), (int)(ru.x + (w - wlo) + extra));
    // the second run, when it is the next head's (which then starts at slot S_u + runs_u)
    int4 second = make_int4(-1, 0, 0, left);
    if (left > 0 && u + 1 < units) {
      const int cn = min(max(a.piv_count[u + 1], 0), a.cap);
      const int t2 = min((cn + PIVOT_CHUNK - 1) / PIVOT_CHUNK, left);
      if (t2 > 0) second = make_int4(u + 1, min(cn, t2 * PIVOT_CHUNK), ru.x + ru.y, left - t2);
    }
    a.sched[2 * w + 1] = second;
  }
}

__global__ __launch_bounds__(UN_NT) void k_piv_schedule(PlanArgs a) { pivot_schedule(a); }

__global__ __launch_bounds__(UN_NT) void k_union(UnionArgs a) {
  if (blockIdx.x == a.t.B * a.t.Hkv) {          // the extra column: the schedule
    if (blockIdx.y == 0) {
      PlanArgs pa;
      pa.t = a.t;
      pa.piv_count = a.piv_count;
      pa.cap = a.cap;
      pa.workers = a.piv_workers;
      pa.sched = a.piv_sched;
      pa.runs = a.piv_runs;
      pivot_schedule(pa);
    }
    return;
  }
  const int unit = blockIdx.x;
  const int b = unit / a.t.Hkv;
  const int g = unit % a.t.Hkv;
  const int G = a.t.G;
  const int Hq = a.t.Hkv * G;
  const int tid = threadIdx.x;
  const uint32_t *fb = a.fbits + word_base(a.t, b, g);
  const int cnt = min(a.piv_count[unit], a.cap);
  const int p = blockIdx.y * UN_NT + tid;
  if (p >= cnt) return;
  const double kappa = a.params[0];
  const int tok = a.piv_idx[(int64_t)unit * a.cap + p];
  if (tok < 0 || tok >= a.t.s[b].n) {
    // a pivot list verkv_compress did not write: weight 0, and no read at that token
    for (int j = 0; j < G; ++j) a.coef[((int64_t)unit * a.cap + p) * G + j] = 0.0f;
    return;
  }
  const double ri = a.r[tok_base(a.t, b, g) + tok];
  const bool exact = (ri >= 1.0) || ((fb[tok >> 5] >> (tok & 31)) & 1);
  for (int j = 0; j < G; ++j) {
    const int h = g * G + j;
    float cf32 = 1.0f;
    if (!exact) {
      const double wi = a.wc[row_tok_base(a.t, b, h) + tok] *
                        a.cscale[row_chunk_base(a.t, b, h) + tok / SKETCH_CHUNK];
      const double lam = lam_of(wi, ri, a.beta_star[(int64_t)b * Hq + h], kappa);
      cf32 = (float)(lam / ri);
    }
    a.coef[((int64_t)unit * a.cap + p) * G + j] = cf32;
  }
}

// ------------------------------------------------------------------ eps_hat(L \ F)
// Partial certificate terms of the tokens that stay sampled, per (row, slice); the
// finishing kernel combines the slices in order (Lemma 1 on L \ F, lambda frozen).
__global__ __launch_bounds__(DC_NT) void k_after(AfterArgs a) {
  __shared__ double scr[4 * DC_NW];
  const int T = a.team;
  const int row = blockIdx.x / T;
  const int m = blockIdx.x % T;
  const int Hq = a.t.Hkv * a.t.G;
  const int b = row / Hq;
  const int h = row % Hq;
  const int g = h / a.t.G;
  const int n = a.t.s[b].n;
  const int s0 = (int)((int64_t)n * m / T);
  const int s1 = (int)((int64_t)n * (m + 1) / T);
  const double *wcr = a.wc + row_tok_base(a.t, b, h);
  const double *sc = a.cscale + row_chunk_base(a.t, b, h);
  const double *rr = a.r + tok_base(a.t, b, g);
  const uint32_t *fb = a.fbits + word_base(a.t, b, g);
  const double Bst = a.beta_star[row];
  const double kappa = a.params[0];
  Cert c{0.0, 0.0, 0.0, 0.0};
  int cnt = 0;
  for (int i = s0 + threadIdx.x; i < s1; i += DC_NT) {
    const double ri = rr[i];
    if (!(ri < 1.0)) continue;
    if ((fb[i >> 5] >> (i & 31)) & 1) continue;
    const double wi = wcr[i] * sc[i / SKETCH_CHUNK];
    const Terms x = terms_of(wi, ri, lam_of(wi, ri, Bst, kappa));
    c.beta += x.beta; c.V += x.V; ++cnt;
    top2_merge(c.b1, c.b2, x.b, 0.0);
  }
  const Cert o = block_cert(c, scr);
  const double tot = block_sum<DC_NT>((double)cnt, scr);
  if (threadIdx.x == 0) {
    double *p = a.part + ((int64_t)row * T + m) * 8;
    p[0] = o.beta; p[1] = o.V; p[2] = o.b1; p[3] = o.b2; p[4] = tot;
  }
}

// ------------------------------------------------------------------ finish a row
// N_hat and D_hat are the fixed-order sums of the partials of the resident pivots and
// of the host rows; o = N_hat / D_hat, lse = m_hat + ln D_hat; eps_after combines the
// slices of k_after.
constexpr int FI_GRP = 4;                  // split groups summed in parallel
constexpr int FI_NT = 576;                 // FI_GRP x (D + 1) = 516 active threads

__global__ __launch_bounds__(FI_NT) void k_finish(FinishArgs a) {
  __shared__ float s_acc[FI_GRP][D + 1];
  __shared__ float s_d;
  const int row = blockIdx.x;
  const int Hq = a.t.Hkv * a.t.G;
  const int b = row / Hq;
  const int h = row % Hq;
  const int g = h / a.t.G;
  const int j = h % a.t.G;
  const int unit = b * a.t.Hkv + g;
  const int tid = threadIdx.x;
  constexpr int PS = D + 1;
  // group q sums the pivot partials [S + q runs/4, S + (q+1) runs/4) and the host
  // splits [q nsh/4, (q+1) nsh/4), 16 loads in flight; the groups are then added in order
  constexpr int FB = 16;
  auto add_parts = [&](const float *base, int s0, int s1, float acc) -> float {
    const int64_t stride = (int64_t)a.t.G * PS;
    for (int sa = s0; sa < s1; sa += FB) {
      float v[FB];
#pragma unroll
      for (int u = 0; u < FB; ++u) v[u] = sa + u < s1 ? base[(sa + u) * stride] : 0.0f;
#pragma unroll
      for (int u = 0; u < FB; ++u)
        if (sa + u < s1) acc += v[u];
    }
    return acc;
  };
  if (tid < FI_GRP * PS) {
    const int q = tid / PS, col = tid % PS;
    float part = 0.0f;
    const int4 rn = a.piv_runs[unit];
    part = add_parts(a.piv_part + ((int64_t)rn.x * a.t.G + j) * PS + col,
                     rn.y * q / FI_GRP, rn.y * (q + 1) / FI_GRP, part);
    part = add_parts(a.host_part + ((int64_t)unit * a.nsh * a.t.G + j) * PS + col,
                     a.nsh * q / FI_GRP, a.nsh * (q + 1) / FI_GRP, part);
    s_acc[q][col] = part;
  }
  __syncthreads();
  float acc = 0.0f;
  if (tid <= D) {
#pragma unroll
    for (int q = 0; q < FI_GRP; ++q) acc += s_acc[q][tid];
    if (tid == D) s_d = acc;
  }
  __syncthreads();
  const float dh = s_d;
  if (tid < D) {
    a.n_hat[(int64_t)row * D + tid] = acc;
    a.o[(int64_t)row * D + tid] = acc / dh;
  } else if (tid == D) {
    a.d_hat[row] = dh;
    a.lse[row] = (float)(a.m_hat[row] + log((double)dh));
  } else if (tid == D + 1) {
    Cert c{0.0, 0.0, 0.0, 0.0};
    double tot = 0.0;
    for (int k = 0; k < a.team; ++k) {
      const double *p = a.after_part + ((int64_t)row * a.team + k) * 8;
      c = cert_combine(c, Cert{p[0], p[1], p[2], p[3]});
      tot += p[4];
    }
    a.eps_after[row] = tot > 0.0 ? bern_E(c.beta, c.V, c.b1, a.params[1]) / a.d_sketch[row] : 0.0;
  }
}

size_t decide_lds_bytes(int nch_max, bool slice_cache) {
  return sizeof(double) * ((size_t)nch_max + (slice_cache ? 4 * (size_t)LDS_TOK : 0));
}

bool decide_slice_cached(int max_n, int team) { return (max_n + team - 1) / team <= LDS_TOK; }

hipError_t launch_decide(DecideArgs &a, int rows, hipStream_t st) {
  // allow the largest dynamic LDS this kernel asks for (chunk scales + slice cache), once
  // per device (the attribute belongs to the kernel as loaded on the current device)
  constexpr int MAX_DEV = 64;
  static std::atomic<bool> attr_set[MAX_DEV];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute((const void *)k_decide, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)std::max(decide_lds_bytes(MAX_CHUNKS, false),
                                          decide_lds_bytes(MAX_CACHED_CHUNKS, true)));
    if (e != hipSuccess) return e;
    attr_set[dev].store(true, std::memory_order_release);
  }
  a.nch_max = chunks_of(a.t.max_n);
  a.lds_cache = decide_slice_cached(a.t.max_n, a.team) ? 1 : 0;
  const size_t dyn = decide_lds_bytes(a.nch_max, a.lds_cache != 0);
  const dim3 grid(rows * a.team), block(DC_NT);
  // An ordinary launch: the caller sizes the grid to what the device holds at once
  // (decide_blocks_per_cu x CUs), so every team is co-resident once earlier work on
  // the stream has drained; a barrier wait that cannot complete still ends (bounded
  // spin, status bit 4).  This avoids the cooperative launch's fixed cost per step.
  return launch_kernel(k_decide, grid, block, (uint32_t)dyn, st, a);
}

int decide_blocks_per_cu(int max_n, int team) {
  const size_t dyn = decide_lds_bytes(chunks_of(max_n), decide_slice_cached(max_n, team));
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_decide, DC_NT, dyn) != hipSuccess) return 1;
  return nb > 0 ? nb : 1;
}

hipError_t launch_union(const UnionArgs &a, int units, hipStream_t st) {
  if (!a.coef_pass) return launch_kernel(k_lists, dim3(LS_NB, units), dim3(LS_NT), 0, st, a);
  return launch_kernel(k_union, dim3(units + (a.piv_sched ? 1 : 0), (a.cap + UN_NT - 1) / UN_NT),
                       dim3(UN_NT), 0, st, a);
}

hipError_t launch_pivot_schedule(const PlanArgs &a, hipStream_t st) {
  return launch_kernel(k_piv_schedule, dim3(1), dim3(UN_NT), 0, st, a);
}

hipError_t launch_after(const AfterArgs &a, int rows, hipStream_t st) {
  return launch_kernel(k_after, dim3(rows * a.team), dim3(DC_NT), 0, st, a);
}

hipError_t launch_finish(const FinishArgs &a, int rows, hipStream_t st) {
  return launch_kernel(k_finish, dim3(rows), dim3(FI_NT), 0, st, a);
}

}  // namespace verkv
