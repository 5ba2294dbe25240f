// KVFetch steps 3-4 for gfx950 with lambda re-solved on every candidate set ("Verify
// Before You Fetch", picx.dev summary page, "KVFETCH" steps 3-4, eqs. (9)-(10)).  Eq. (9)
// writes eps_hat(L \ {i}) without saying whether the shrinkage bias of Definition 2
// follows the set; this kernel takes the reading where it does on the cut of step 4:
// the order is eq. (9)'s g with lambda frozen at the full L (the decision kernel's
// keys, rebuilt here bit for bit), and k* is the least k for which eps_hat of L_g[k:],
// with the bias solved on L_g[k:] alone, is below eps.  The kept set keeps that bias.
//
// eps_hat of L_g[k:] so defined is non-increasing in k: a subset's bias function lies
// below its parent's at every B, so its fixed point is no larger; lambda, V_i and b_i
// grow with B; and eq. (7)'s numerator grows with the bias, V and b.  So k* is the
// boundary of a monotone predicate and is found by search, not a scan.  The candidate
// sets are {tokens whose extended key (g, reversed index) is below a threshold}; the
// search descends the same digits of the key as the frozen reading's k* search: at
// each level the counts of the current window per digit (merged over the team) give
// the non-empty buckets, a binary search over their lower boundaries finds the bucket
// in which the predicate turns false, and the window moves into it; once at most WIN
// tokens remain they are sorted and a binary search over them finds the cut token.
// Every probe solves the bias exactly on its set (the safeguarded Newton iteration of
// the decision kernel, exact on the final linear piece), started from the neighbouring
// probes' solutions, and evaluates eq. (7) on that piece.
#include "decide_util.h"

#include <algorithm>
#include <atomic>

namespace verkv {

constexpr uint32_t XBASE = 1u << 20;       // exchange numbers of this kernel start here

__global__ __launch_bounds__(DC_NT) void k_resolve(ResolveArgs a) {
  extern __shared__ double s_dyn[];          // [nch] chunk scales, then [4][LDS_TOK] cache
  __shared__ double scr[NQ * DC_NW];
  __shared__ double s_part[TEAM_MAX * PART];
  __shared__ uint32_t h_cnt[NBUCKET];
  __shared__ int32_t s_nb[NBUCKET];
  __shared__ uint64_t w_key[WIN];
  __shared__ uint32_t w_lo[WIN];
  __shared__ int32_t s_int[4];
  __shared__ int32_t iscr[DC_NW];

  const int T = a.team;
  int row, m;
  if (a.xcd_map) {
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
  if (a.certified[row]) return;              // the whole team: no fetch for this row
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
  const bool cached = (s1 - s0) <= TR * DC_NT;
  const bool lcache = (s1 - s0) <= LDS_TOK && a.lds_cache;
  double *s_scale = s_dyn;
  double *s_w = s_dyn + a.nch_max;
  double *s_r = s_w + LDS_TOK;
  double *s_ir = s_r + LDS_TOK;
  double *s_rq = s_ir + LDS_TOK;
  const double *wcr = a.wc + row_tok_base(a.t, b, h);
  const double *rr = a.r + tok_base(a.t, b, g);
  uint32_t *fb = a.fbits + word_base(a.t, b, g);
  const double kappa = a.kappa, l = a.l, eps = a.eps;
  const double Dd = a.d_sketch[row];
  const double Bfull = a.beta_star[row];     // bias of the full L (read before any exchange)
  const double V = a.gpar[4 * row], b1 = a.gpar[4 * row + 1], b2 = a.gpar[4 * row + 2];
  const double sqX = a.gpar[4 * row + 3];
  const double kB = kappa * Bfull;
  const int TW = a.team_ws;
  double *xseq = a.xseq + (int64_t)row * 2 * TW;
  double *part = a.part + (int64_t)row * 2 * TW * PART;
  uint32_t nx = XBASE;
#define XPAR() ((int)((nx + 1) & 1))
#define TEAM_SYNC()                                                         \
  do {                                                                      \
    if (T > 1) { ++nx; team_exchange(xseq + (nx & 1) * TW, m, T, nx, a.status); } \
    else __syncthreads();                                                   \
  } while (0)
#define SLOT() (part + (int64_t)XPAR() * TW * PART)
#define TEAM_STAGE(sl)                                                      \
  do {                                                                      \
    TEAM_SYNC();                                                            \
    for (int j_ = tid; j_ < T * PART; j_ += DC_NT) s_part[j_] = xget((sl) + j_); \
    __syncthreads();                                                        \
  } while (0)

  double rb0[TR], wb0[TR];                   // the slice, loaded ahead (LDS cache only)
  if (lcache) {
#pragma unroll
    for (int k = 0; k < TR; ++k) {
      const int i = s0 + tid + k * DC_NT;
      rb0[k] = i < s1 ? rr[i] : 2.0;
      wb0[k] = i < s1 ? wcr[i] : 0.0;
    }
  }
  // chunk scales exp(m_c - m_hat) (the decision kernel's), f(0) of the full L
  const double *cs = a.cscale + row_chunk_base(a.t, b, h);
  const double *cz = a.cf0 + row_chunk_base(a.t, b, h);
  double zloc = 0.0;
  for (int c = tid; c < nch; c += DC_NT) {
    s_scale[c] = cs[c];
    zloc += cs[c] * cz[c];
  }
  const double f0 = block_sum<DC_NT>(zloc, scr);   // its barrier also publishes s_scale
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
  const bool kinf = isinf(kappa);
  // the fetch key of eq. (9) with lambda frozen, exactly as the decision kernel forms it
  auto key_of = [&](double wi, double ri, double ir, double rq) -> uint64_t {
    const Terms x = terms_at(wi, ri, ir, rq, kB, kinf);
    return dbits(g_of(x, V, b1, b2, l, Dd, sqX));
  };
  uint64_t ckey[TR];
#pragma unroll
  for (int k = 0; k < TR; ++k) {
    ckey[k] = 0;
    const int i = s0 + tid + k * DC_NT;
    if (cached && i < s1) {
      const double ri = lcache ? s_r[i - s0] : rr[i];
      if (ri < 1.0) {
        const double wi = lcache ? s_w[i - s0] : wcr[i] * s_scale[i / SKETCH_CHUNK];
        const double ir = lcache ? s_ir[i - s0] : (ri > 0.0 ? 1.0 / ri : 0.0);
        const double rq = lcache ? s_rq[i - s0] : ri / (1.0 - ri);
        ckey[k] = key_of(wi, ri, ir, rq);
      }
    }
  }
  // every token of L in this member's slice: ri, wi, ir, rq, key, lo
#define FOR_T(body)                                                            \
  if (cached) {                                                                \
    _Pragma("unroll")                                                          \
    for (int k = 0; k < TR; ++k) {                                             \
      const int i = s0 + tid + k * DC_NT;                                      \
      if (i >= s1) continue;                                                   \
      const double ri = lcache ? s_r[i - s0] : rr[i];                          \
      if (!(ri < 1.0)) continue;                                               \
      const double wi = lcache ? s_w[i - s0] : wcr[i] * s_scale[i / SKETCH_CHUNK]; \
      const double ir = lcache ? s_ir[i - s0] : (ri > 0.0 ? 1.0 / ri : 0.0);   \
      const double rq = lcache ? s_rq[i - s0] : ri / (1.0 - ri);               \
      const uint64_t key = ckey[k];                                            \
      const uint32_t lo = IDX_MAX - (uint32_t)i;                               \
      body                                                                     \
    }                                                                          \
  } else {                                                                     \
    for (int i = s0 + tid; i < s1; i += DC_NT) {                               \
      const double ri = rr[i];                                                 \
      if (!(ri < 1.0)) continue;                                               \
      const double wi = wcr[i] * s_scale[i / SKETCH_CHUNK];                    \
      const double ir = ri > 0.0 ? 1.0 / ri : 0.0;                             \
      const double rq = ri / (1.0 - ri);                                       \
      const uint64_t key = key_of(wi, ri, ir, rq);                             \
      const uint32_t lo = IDX_MAX - (uint32_t)i;                               \
      body                                                                     \
    }                                                                          \
  }

  // A probe: the bias of Definition 2 solved on S = {tokens of L with (key, lo) below
  // (tk, tl)} by the safeguarded Newton iteration, started at `start`, and whether
  // eps_hat(S) of eq. (7) on the final piece is below eps.  Every member takes the same
  // path (team-combined values in member order).
  const double inv_kappa = 1.0 / kappa;
  auto probe = [&](uint64_t tk, uint32_t tl, double start, double &Bout) -> bool {
    if (kinf || kappa == 0.0) {
      // lambda is 1 (kappa infinite) or r (kappa 0) whatever the bias: one pass gives the
      // bias of S (the sum of w (1 - lambda)) and eq. (7)'s totals
      Cert c{0.0, 0.0, 0.0, 0.0};
      double cnt = 0.0;
      FOR_T(
        if (key < tk || (key == tk && lo < tl)) {
          const Terms x = terms_at(wi, ri, ir, rq, 0.0, kinf);
          c.beta += x.beta; c.V += x.V; cnt += 1.0;
          top2_merge(c.b1, c.b2, x.b, 0.0);
        })
      c = block_cert(c, scr);
      cnt = block_sum<DC_NT>(cnt, scr);
      if (T > 1) {
        double *sl = SLOT();
        if (tid == 0) {
          double *q = sl + m * PART;
          xput(q + 0, c.beta); xput(q + 1, c.V); xput(q + 2, c.b1); xput(q + 3, c.b2); xput(q + 4, cnt);
        }
        TEAM_STAGE(sl);
        c = Cert{0.0, 0.0, 0.0, 0.0};
        cnt = 0.0;
        for (int k = 0; k < T; ++k) {
          const double *q = s_part + k * PART;
          c = cert_combine(c, Cert{q[0], q[1], q[2], q[3]});
          cnt += q[4];
        }
        __syncthreads();
      }
      Bout = c.beta;
      const double E = cnt > 0.0 ? bern_E(c.beta, c.V, c.b1, l) : 0.0;
      return E / Dd < eps;
    }
    double lo_b = 0.0, hi_b = f0;
    double B = fmin(fmax(start, 0.0), f0);
    bool eval_only = false;          // one more pass at B for the totals, no further step
    for (int iter = 0; iter < 201; ++iter) {
      NewtonAcc v{0.0, 0.0, 0.0, INFINITY, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
      FOR_T(
        if (key < tk || (key == tk && lo < tl)) newton_add(v, ri, wi, ir, rq, B, kappa, inv_kappa);)
      // the step needs the linear model and its piece; the eq. (7) totals of the pass
      // are reduced once the root lies on that piece
      Lin lm = block_lin(v, scr);
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
        __syncthreads();
      }
      const double hB = B * (1.0 + lm.c1) - lm.c0;
      double Bn = lm.c0 / (1.0 + lm.c1);
      bool on_piece = (Bn >= lm.lo && Bn <= lm.hi);
      if (!on_piece && hB == 0.0) { Bn = B; on_piece = true; }
      if (eval_only) { Bn = B; on_piece = true; }  // the model of B's own piece, at B
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
          __syncthreads();
        }
        // eq. (7) on this piece at Bn: bias c0 - Bn c1, V = vc + Bn^2 vm, b the larger of
        // the constant b_i and Bn times the largest mid-piece coefficient
        Bout = Bn;
        double c1 = o.bc1, c2 = o.bc2;
        top2_merge(c1, c2, Bn * o.bm1, Bn * o.bm2);
        const double E = o.cnt > 0.0 ? bern_E(o.c0 - Bn * o.c1, o.vc + Bn * Bn * o.vm, c1, l) : 0.0;
        return E / Dd < eps;
      }
      if (hB < 0.0) lo_b = B; else hi_b = B;
      double Bnext = Bn;
      if (!(Bnext > lo_b && Bnext < hi_b)) Bnext = 0.5 * (lo_b + hi_b);
      if (Bnext == B || !(hi_b > lo_b) || iter >= 199) {
        // no further progress: take the totals at the last piece root, as the decision
        // kernel does (flagged only when the iteration count ran out)
        if (iter >= 199 && tid == 0 && m == 0) atomicOr(a.status, 2);
        B = Bn;
        eval_only = true;
        continue;
      }
      B = Bnext;
    }
    Bout = B;
    return false;
  };

  // ---- the descent over the digits of the key
  double Blo = 0.0, Bhi = Bfull;       // biases of the kept-so-far set (certifies) and of
                                       // it with the window (does not)
  uint64_t pkey = 0;
  uint32_t plo = 0;
  int lev = -1;
  auto in_window = [&](uint64_t key, uint32_t lo) { return cmp_window(key, lo, lev, pkey, plo) == 0; };
  int wcnt = 0;
  for (int L = 0; L < NLEV; ++L) {
    for (int k = tid; k < NBUCKET; k += DC_NT) h_cnt[k] = 0;
    __syncthreads();
    const int sh = c_lev_shift[L];
    const uint32_t dmask = (1u << c_lev_width[L]) - 1u;
    FOR_T(
      if (in_window(key, lo)) {
        const uint32_t dig = c_lev_lo[L] ? ((lo >> sh) & dmask) : (uint32_t)((key >> sh) & dmask);
        atomicAdd(&h_cnt[dig], 1u);
      })
    __syncthreads();
    if (T > 1) {
      const int64_t hp = (int64_t)row * 2 * TW * NBUCKET + (int64_t)XPAR() * TW * NBUCKET;
      for (int k = tid; k < NBUCKET; k += DC_NT) xput(a.hcnt + hp + (int64_t)m * NBUCKET + k, h_cnt[k]);
      TEAM_SYNC();
      for (int k = tid; k < NBUCKET; k += DC_NT) {
        uint32_t c = 0;
        for (int q = 0; q < T; ++q) c += xget(a.hcnt + hp + (int64_t)q * NBUCKET + k);
        h_cnt[k] = c;
      }
      __syncthreads();
    }
    // the non-empty buckets in ascending digit order
    const int mycnt = tid < NBUCKET ? (int)h_cnt[tid] : 0;
    int32_t nnz = 0;
    const int32_t pos = block_excl_scan<DC_NT>(mycnt > 0 ? 1 : 0, iscr, &nnz);
    if (mycnt > 0) s_nb[pos] = tid;
    __syncthreads();
    if (nnz == 0) break;                 // an empty window: nothing left to split
    // S(i) = kept-so-far plus the buckets below s_nb[i]: S(0) certifies, the whole
    // window (i = nnz) does not; find the last i that certifies
    int ilo = 0, ihi = nnz;
    while (ihi - ilo > 1) {
      const int mid = (ilo + ihi) >> 1;
      const uint32_t j = (uint32_t)s_nb[mid];
      uint64_t tk;
      uint32_t tl;
      if (!c_lev_lo[L]) {
        tk = ((L == 0 ? 0ull : (pkey << c_lev_width[L])) | (uint64_t)j) << sh;
        tl = 0;
      } else {
        tk = pkey;
        tl = ((L == FIRST_LO_LEV ? 0u : (plo << c_lev_width[L])) | j) << sh;
      }
      double Bt = 0.0;
      if (probe(tk, tl, Bhi, Bt)) { ilo = mid; Blo = Bt; } else { ihi = mid; Bhi = Bt; }
    }
    const uint32_t jstar = (uint32_t)s_nb[ilo];
    wcnt = (int)h_cnt[jstar];
    if (!c_lev_lo[L]) pkey = (L == 0) ? (uint64_t)jstar : ((pkey << c_lev_width[L]) | (uint64_t)jstar);
    else plo = (L == FIRST_LO_LEV) ? jstar : ((plo << c_lev_width[L]) | jstar);
    lev = L;
    __syncthreads();
    if (wcnt <= WIN) break;
  }

  // ---- the last window (at most WIN tokens): gather, sort ascending, binary search
  if (tid == 0) s_int[1] = 0;
  for (int k = tid; k < WIN; k += DC_NT) { w_key[k] = ~0ull; w_lo[k] = ~0u; }
  __syncthreads();
  uint64_t *gkey = a.wkey + (int64_t)row * WIN;
  uint32_t *glo = a.wlo + (int64_t)row * WIN;
  FOR_T(
    if (in_window(key, lo)) {
      if (T > 1) {
        const uint32_t p = atomicAdd(&a.wcount[row], 1u);
        if (p < (uint32_t)WIN) { xput(gkey + p, key); xput(glo + p, lo); }
      } else {
        const int p = atomicAdd(&s_int[1], 1);
        if (p < WIN) { w_key[p] = key; w_lo[p] = lo; }
      }
    })
  if (T > 1) {
    TEAM_SYNC();
    const int wc = min((int)__hip_atomic_load(&a.wcount[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), WIN);
    for (int k = tid; k < wc; k += DC_NT) { w_key[k] = xget(gkey + k); w_lo[k] = xget(glo + k); }
    if (tid == 0) s_int[1] = wc;
    __syncthreads();
  }
  __syncthreads();
  const int wc = min(s_int[1], WIN);
  {
    int P = 2;
    while (P < wc) P <<= 1;
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
  }
  // S(p) = {ext below window token p}: S(0) is the kept-so-far set (certifies), the
  // whole window (p = wc) does not; the cut token is window token plast
  int plast = 0, phi = wc;
  while (phi - plast > 1) {
    const int mid = (plast + phi) >> 1;
    double Bt = 0.0;
    if (probe(w_key[mid], w_lo[mid], Bhi, Bt)) { plast = mid; Blo = Bt; } else { phi = mid; Bhi = Bt; }
  }
  const uint64_t tkey = w_key[plast];
  const uint32_t tlo = w_lo[plast];
  __syncthreads();

  // ---- F_h = tokens at or above the cut token in the extended key
  int64_t kc = 0;
  if (cached) {
#pragma unroll
    for (int k = 0; k < TR; ++k) {
      const int i = s0 + tid + k * DC_NT;
      bool f = false;
      if (i < s1) {
        const double ri = lcache ? s_r[i - s0] : rr[i];
        const uint32_t lo = IDX_MAX - (uint32_t)i;
        f = ri < 1.0 && (ckey[k] > tkey || (ckey[k] == tkey && lo >= tlo));
      }
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
          const uint64_t key = key_of(wi, ri, ri > 0.0 ? 1.0 / ri : 0.0, ri / (1.0 - ri));
          const uint32_t lo = IDX_MAX - (uint32_t)i;
          f = key > tkey || (key == tkey && lo >= tlo);
        }
      }
      kc += f ? 1 : 0;
      or_bits_wave(fb, i - lane, f, lane);
    }
  }
  const int64_t ks = block_sum_i64<DC_NT>(kc, (int64_t *)scr);
  if (tid == 0 && ks) atomicAdd(&a.kstar[row], (int32_t)ks);
  // the kept set keeps the bias solved on it
  if (tid == 0 && m == 0) a.beta_star[row] = Blo;
#undef FOR_T
#undef TEAM_STAGE
#undef TEAM_SYNC
#undef SLOT
#undef XPAR
}

static size_t resolve_lds_bytes(int nch_max, bool slice_cache) {
  return sizeof(double) * ((size_t)nch_max + (slice_cache ? 4 * (size_t)LDS_TOK : 0));
}

hipError_t launch_resolve(ResolveArgs &a, int rows, hipStream_t st) {
  constexpr int MAX_DEV = 64;
  static std::atomic<bool> attr_set[MAX_DEV];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute((const void *)k_resolve, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)std::max(resolve_lds_bytes(MAX_CHUNKS, false),
                                          resolve_lds_bytes(MAX_CACHED_CHUNKS, true)));
    if (e != hipSuccess) return e;
    attr_set[dev].store(true, std::memory_order_release);
  }
  const size_t dyn = resolve_lds_bytes(a.nch_max, a.lds_cache != 0);
  return launch_kernel(k_resolve, dim3(rows * a.team), dim3(DC_NT), (uint32_t)dyn, st, a);
}

int resolve_blocks_per_cu(int nch_max, bool slice_cache) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_resolve, DC_NT,
                                                   resolve_lds_bytes(nch_max, slice_cache)) != hipSuccess)
    return 1;
  return nb > 0 ? nb : 1;
}

}  // namespace verkv
