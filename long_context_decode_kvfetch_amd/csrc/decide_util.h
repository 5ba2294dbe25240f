// Device helpers of the KVFetch decision kernels (steps 2-4 in float64): the
// estimator terms of Definition 2, the eq. (7) numerator, the eq. (9) fetch priority,
// the digit windows of the k* search, fixed-order block reductions and the team
// exchange.  Included by the decision kernel files only.
#pragma once
#include "kernels.h"

namespace verkv {

constexpr int DC_NT = DECIDE_THREADS;
constexpr int DC_NW = DC_NT / WAVE;
constexpr int MAX_CHUNKS = VERKV_MAX_SEQ_LEN / SKETCH_CHUNK;
constexpr uint32_t IDX_MAX = (1u << 20) - 1;
// digit levels: 7 of the 63 bits of g >= 0 (9 bits each), then 3 of the 20-bit
// tie-breaking token key
constexpr int NLEV = 10;
constexpr int FIRST_LO_LEV = 7;
static __device__ __constant__ int c_lev_lo[NLEV] = {0, 0, 0, 0, 0, 0, 0, 1, 1, 1};
static __device__ __constant__ int c_lev_shift[NLEV] = {54, 45, 36, 27, 18, 9, 0, 11, 2, 0};
static __device__ __constant__ int c_lev_width[NLEV] = {9, 9, 9, 9, 9, 9, 9, 9, 9, 2};

__device__ __forceinline__ double lam_of(double w, double r, double B, double kappa) {
  if (r == 0.0) return 0.0;
  if (w == 0.0) return 1.0;
  if (isinf(kappa)) return 1.0;
  const double x = (kappa * B * r) / (w * (1.0 - r));
  return fmin(1.0, fmax(r, x));
}

struct Terms { double beta, V, b; };
__device__ __forceinline__ Terms terms_of(double w, double r, double lam) {
  Terms t;
  t.beta = w * (1.0 - lam);
  if (r > 0.0) {
    t.V = lam * lam * w * w * (1.0 - r) / r;
    t.b = lam * w * fmax(r, 1.0 - r) / r;
  } else {
    t.V = 0.0;
    t.b = 0.0;
  }
  return t;
}

// terms_of(w, r, lam_of(w, r, B, kappa)) written with 1/r (ir) and r/(1-r) (rq) at
// hand: lambda w is kB rq on the middle piece, so every term is a product.
__device__ __forceinline__ Terms terms_at(double w, double r, double ir, double rq, double kB,
                                          bool kinf) {
  Terms t{0.0, 0.0, 0.0};
  if (r == 0.0) { t.beta = w; return t; }             // lambda = 0
  if (w == 0.0) return t;                             // lambda = 1, nothing left
  const double q1 = 1.0 - r, mx = fmax(r, q1);
  const double num = kinf ? INFINITY : kB * rq;       // lambda w before the clip
  if (num >= w) {                                     // lambda = 1
    t.V = w * w * q1 * ir;
    t.b = w * mx * ir;
  } else if (num <= r * w) {                          // lambda = r
    t.beta = w * q1;
    t.V = r * w * w * q1;
    t.b = w * mx;
  } else {                                            // lambda w = kB rq
    t.beta = w - num;
    t.V = num * num * q1 * ir;
    t.b = num * mx * ir;
  }
  return t;
}

__device__ __forceinline__ double bern_E(double beta, double V, double b, double l) {
  const double t = b * l / 3.0;
  return beta + t + sqrt(t * t + 2.0 * V * l);
}

// g_i of eq. (9), lambda frozen; sqrt(X) - sqrt(Y) evaluated as (X - Y)/(sqrt X + sqrt Y).
// sqX = sqrt(X) with X = (b1 l/3)^2 + 2 V l is the same for every token of the row.
__device__ __forceinline__ double g_of(const Terms &x, double V, double b1, double b2, double l,
                                       double Dd, double sqX) {
  const double bm = (x.b == b1) ? b2 : b1;
  const double t1 = b1 * l / 3.0, tm = bm * l / 3.0;
  const double Y = tm * tm + 2.0 * (V - x.V) * l;
  const double dX = (t1 - tm) * (t1 + tm) + 2.0 * x.V * l;
  const double den = sqX + sqrt(Y);
  const double frac = den > 0.0 ? dX / den : 0.0;
  const double g = (x.beta + (t1 - tm) + frac) / Dd;
  return g > 0.0 ? g : 0.0;                     // maps -0 to +0
}

__device__ __forceinline__ uint64_t dbits(double v) { return (uint64_t)__double_as_longlong(v); }
__device__ __forceinline__ double bitsd(uint64_t v) { return __longlong_as_double((long long)v); }

// Position of the extended key (key, lo) relative to the window "prefix P at level lev":
// -1 below, 0 inside, +1 above.  lev < 0 is the whole set.
__device__ __forceinline__ int cmp_window(uint64_t key, uint32_t lo, int lev, uint64_t pkey,
                                          uint32_t plo) {
  if (lev < 0) return 0;
  if (!c_lev_lo[lev]) {
    const uint64_t kp = key >> c_lev_shift[lev];
    return kp < pkey ? -1 : (kp > pkey ? 1 : 0);
  }
  if (key != pkey) return key < pkey ? -1 : 1;
  const uint32_t lp = lo >> c_lev_shift[lev];
  return lp < plo ? -1 : (lp > plo ? 1 : 0);
}

// Four fixed-order block reductions in one barrier round (see block_sum).
struct Red4 { double s0, s1, mx, mn; };
__device__ __forceinline__ Red4 block_red4(Red4 v, double *scr /*[4*DC_NW]*/) {
  v.s0 = wave_sum(v.s0);
  v.s1 = wave_sum(v.s1);
  v.mx = wave_max(v.mx);
  v.mn = wave_min(v.mn);
  const int w = threadIdx.x / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  if (lane == 0) {
    scr[w] = v.s0; scr[DC_NW + w] = v.s1; scr[2 * DC_NW + w] = v.mx; scr[3 * DC_NW + w] = v.mn;
  }
  __syncthreads();
  const int k = lane & 15;
  const bool in = k < DC_NW;
  Red4 o;
  o.s0 = sum16(in ? scr[k] : 0.0);
  o.s1 = sum16(in ? scr[DC_NW + k] : 0.0);
  o.mx = max16(in ? scr[2 * DC_NW + k] : -INFINITY);
  o.mn = min16(in ? scr[3 * DC_NW + k] : INFINITY);
  __syncthreads();
  return o;
}

// Sums of beta and V, the maximum b and the runner-up b (multiset), fixed order.
struct Cert { double beta, V, b1, b2; };
__device__ __forceinline__ void top2_merge(double &a1, double &a2, double c1, double c2) {
  const double hi = fmax(a1, c1);
  const double lo2 = fmax(fmin(a1, c1), fmax(a2, c2));
  a1 = hi;
  a2 = lo2;
}
template <int CTRL>
__device__ __forceinline__ void top2_step_dpp(double &a1, double &a2) {
  const double c1 = dpp_d<CTRL>(a1), c2 = dpp_d<CTRL>(a2);
  top2_merge(a1, a2, c1, c2);
}
__device__ __forceinline__ void top2_16(double &a1, double &a2) {
  top2_step_dpp<DPP_XOR1>(a1, a2);
  top2_step_dpp<DPP_XOR2>(a1, a2);
  top2_step_dpp<DPP_HALF_MIRROR>(a1, a2);
  top2_step_dpp<DPP_MIRROR>(a1, a2);
}
__device__ __forceinline__ Cert block_cert(Cert v, double *scr /*[4*DC_NW]*/) {
  v.beta = wave_sum(v.beta);
  v.V = wave_sum(v.V);
  top2_16(v.b1, v.b2);
  for (int m = 16; m < WAVE; m <<= 1) {
    const double o1 = shfl_xor_d(v.b1, m), o2 = shfl_xor_d(v.b2, m);
    top2_merge(v.b1, v.b2, o1, o2);
  }
  const int w = threadIdx.x / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  if (lane == 0) {
    scr[w] = v.beta; scr[DC_NW + w] = v.V; scr[2 * DC_NW + w] = v.b1; scr[3 * DC_NW + w] = v.b2;
  }
  __syncthreads();
  const int k = lane & 15;
  const bool in = k < DC_NW;
  Cert o;
  o.beta = sum16(in ? scr[k] : 0.0);
  o.V = sum16(in ? scr[DC_NW + k] : 0.0);
  o.b1 = in ? scr[2 * DC_NW + k] : 0.0;
  o.b2 = in ? scr[3 * DC_NW + k] : 0.0;
  top2_16(o.b1, o.b2);
  __syncthreads();
  return o;
}

// Per-pass accumulator of the Newton iteration for the bias: the linear model of f on
// the piece containing B (C0, C1 and the piece's ends), plus what the certificate
// needs if the root lies on this piece: on a piece every lambda_i is r_i, 1 or
// B kappa r_i / (w_i (1 - r_i)), so V(L) = Vc + B^2 Vm and b(L) is the larger of the
// constant b_i and B times the largest mid-piece coefficient (top two of each kept).
struct NewtonAcc {
  double c0, c1, lo, hi;       // model and piece [lo, hi]
  double vc, vm, cnt;          // V constant part, V coefficient of B^2, |L|
  double bc1, bc2, bm1, bm2;   // top two constant b, top two mid coefficients
};
constexpr int NQ = 11;

// One token of L in a Newton pass at B: lambda = r below aa = w (1 - r) / kappa, 1
// above tt = aa / r, linear in between; with 1/r (ir) and r/(1-r) (rq) at hand every
// term is a product.  Adds the token's piece of the linear model and of the eq. (7)
// totals on that piece.
__device__ __forceinline__ void newton_add(NewtonAcc &v, double ri, double wi, double ir,
                                           double rq, double B, double kappa, double inv_kappa) {
  v.cnt += 1.0;
  if (ri == 0.0) { v.c0 += wi; return; }
  if (wi == 0.0) return;
  const double q1 = 1.0 - ri;
  const double iq = 1.0 + rq;                      // 1 / (1 - r)
  const double wq = wi * q1;
  const double aa = wq * inv_kappa;
  const double tt = aa * ir;
  const double mx = fmax(ri, q1);
  const bool plo = B <= aa;
  const bool phi = !plo && B >= tt;
  const bool pmid = !plo && !phi;
  v.c0 += plo ? wq : (pmid ? wi : 0.0);
  v.c1 += pmid ? kappa * rq : 0.0;
  v.vm += pmid ? kappa * kappa * rq : 0.0;
  v.vc += plo ? ri * wi * wq : (phi ? wi * wq * ir : 0.0);
  v.lo = fmax(v.lo, plo ? 0.0 : (phi ? tt : aa));
  v.hi = fmin(v.hi, plo ? aa : (phi ? INFINITY : tt));
  const double bc = plo ? wi * mx : wi * mx * ir;
  top2_merge(v.bc1, v.bc2, pmid ? 0.0 : bc, 0.0);
  top2_merge(v.bm1, v.bm2, pmid ? kappa * mx * iq : 0.0, 0.0);
}
// The four fields a Newton step needs (the linear model c0 - c1 B of f on the piece and
// the piece's ends), reduced over the block exactly as block_newton reduces them.
struct Lin { double c0, c1, lo, hi; };
__device__ __forceinline__ Lin block_lin(const NewtonAcc &a, double *scr /*[4*DC_NW]*/) {
  double c0 = wave_sum(a.c0), c1 = wave_sum(a.c1);
  double lo = wave_max(a.lo), hi = wave_min(a.hi);
  const int w = threadIdx.x / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  if (lane == 0) {
    double *q = scr + w;
    q[0] = c0; q[DC_NW] = c1; q[2 * DC_NW] = lo; q[3 * DC_NW] = hi;
  }
  __syncthreads();
  const int k = lane & 15;
  const bool in = k < DC_NW;
  const double *q = scr + (in ? k : 0);
  Lin o;
  o.c0 = sum16(in ? q[0] : 0.0); o.c1 = sum16(in ? q[DC_NW] : 0.0);
  o.lo = max16(in ? q[2 * DC_NW] : 0.0); o.hi = min16(in ? q[3 * DC_NW] : INFINITY);
  __syncthreads();
  return o;
}

__device__ __forceinline__ NewtonAcc block_newton(NewtonAcc v, double *scr /*[NQ*DC_NW]*/) {
  v.c0 = wave_sum(v.c0); v.c1 = wave_sum(v.c1);
  v.vc = wave_sum(v.vc); v.vm = wave_sum(v.vm); v.cnt = wave_sum(v.cnt);
  v.lo = wave_max(v.lo); v.hi = wave_min(v.hi);
  top2_16(v.bc1, v.bc2);
  top2_16(v.bm1, v.bm2);
  for (int m = 16; m < WAVE; m <<= 1) {
    double o1 = shfl_xor_d(v.bc1, m), o2 = shfl_xor_d(v.bc2, m);
    top2_merge(v.bc1, v.bc2, o1, o2);
    o1 = shfl_xor_d(v.bm1, m); o2 = shfl_xor_d(v.bm2, m);
    top2_merge(v.bm1, v.bm2, o1, o2);
  }
  const int w = threadIdx.x / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  if (lane == 0) {
    double *q = scr + w;
    q[0] = v.c0; q[DC_NW] = v.c1; q[2 * DC_NW] = v.lo; q[3 * DC_NW] = v.hi;
    q[4 * DC_NW] = v.vc; q[5 * DC_NW] = v.vm; q[6 * DC_NW] = v.cnt;
    q[7 * DC_NW] = v.bc1; q[8 * DC_NW] = v.bc2; q[9 * DC_NW] = v.bm1; q[10 * DC_NW] = v.bm2;
  }
  __syncthreads();
  const int k = lane & 15;
  const bool in = k < DC_NW;
  const double *q = scr + (in ? k : 0);
  NewtonAcc o;
  o.c0 = sum16(in ? q[0] : 0.0); o.c1 = sum16(in ? q[DC_NW] : 0.0);
  o.lo = max16(in ? q[2 * DC_NW] : 0.0); o.hi = min16(in ? q[3 * DC_NW] : INFINITY);
  o.vc = sum16(in ? q[4 * DC_NW] : 0.0); o.vm = sum16(in ? q[5 * DC_NW] : 0.0);
  o.cnt = sum16(in ? q[6 * DC_NW] : 0.0);
  o.bc1 = in ? q[7 * DC_NW] : 0.0; o.bc2 = in ? q[8 * DC_NW] : 0.0;
  o.bm1 = in ? q[9 * DC_NW] : 0.0; o.bm2 = in ? q[10 * DC_NW] : 0.0;
  top2_16(o.bc1, o.bc2);
  top2_16(o.bm1, o.bm2);
  __syncthreads();
  return o;
}

// ------------------------------------------------------------------ team exchange
constexpr uint32_t SPIN_LIMIT = 1u << 24;

// Everything members exchange goes through agent-scope atomic stores and loads, which
// the device keeps coherent across CUs and XCDs without whole-cache write-backs or
// invalidations.  A member publishes exchange k by waiting until its own stores are
// complete, then storing k into its sequence word; it proceeds once every member's
// sequence word reads k.  Sequence words are double-buffered by the parity of k (and
// cleared by the sketch kernel each step), so a member running one exchange ahead
// never overwrites a word or a data slot that a slower member still has to read: to
// write parity p again for exchange k + 2 it must have seen every member publish
// k + 1, which each does only after reading the data of k.  The spin is bounded and
// reports a timeout in the status word instead of hanging.
__device__ __forceinline__ void xput(double *p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void xput(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void xput(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename X>
__device__ __forceinline__ X xget(const X *p) {
  return __hip_atomic_load(const_cast<X *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void team_exchange(double *seq /*[T] of this parity*/, int m, int T,
                                              uint32_t k, int32_t *status) {
  __builtin_amdgcn_s_waitcnt(0);          // this thread's exchange stores are complete
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  const double kd = (double)k;
  if (threadIdx.x == 0) xput(seq + m, kd);
  if (threadIdx.x < (unsigned)T) {
    uint32_t spins = 0;
    while (xget(seq + threadIdx.x) != kd) {
      if (++spins > SPIN_LIMIT) {
        atomicOr(status, 4);
        break;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  __syncthreads();
}

// OR the flags of the wave's 64 consecutive tokens base, base+1, ... into the bitmask:
// one ballot, then lanes 0-2 OR the (at most three) 32-bit words the run touches.
// Every lane of the wave must call it.
__device__ __forceinline__ void or_bits_wave(uint32_t *fb, int base, bool flag, int lane) {
  const uint64_t M = __ballot(flag);
  if (!M) return;
  const int sh = base & 31;
  if (lane < 3) {
    uint32_t v;
    if (lane == 0) v = (uint32_t)(M << sh);
    else if (lane == 1) v = (uint32_t)(M >> (32 - sh));
    else v = sh ? (uint32_t)(M >> (64 - sh)) : 0u;
    if (v) atomicOr(&fb[(base >> 5) + lane], v);
  }
}

__device__ __forceinline__ Cert cert_combine(Cert a, const Cert &b) {
  a.beta += b.beta;
  a.V += b.V;
  top2_merge(a.b1, a.b2, b.b1, b.b2);
  return a;
}

// A member keeps its slice's sketch weights and inclusion probabilities in LDS
// (dynamic shared memory, up to LDS_TOK tokens) for the fixed-point passes, and the
// selection terms and keys of up to TR tokens per thread in registers (slot k of thread
// t is token s0 + t + k * DC_NT).  Longer slices are streamed from memory on every pass,
// four tokens' loads in flight per thread.
constexpr int TR = 8;
constexpr int LDS_TOK = 4096;
// the slice cache is only used when n <= TEAM_MAX * LDS_TOK, which bounds the chunk
// scales that share the dynamic LDS with it
constexpr int MAX_CACHED_CHUNKS = (TEAM_MAX * LDS_TOK + SKETCH_CHUNK - 1) / SKETCH_CHUNK;
constexpr int SB = 4;

// Sort (key, lo) ascending across the 64 lanes of a wave (bitonic, registers only).
__device__ __forceinline__ void wave_bitonic(uint64_t &key, uint32_t &lo) {
  const int lane = threadIdx.x & (WAVE - 1);
  for (int k = 2; k <= WAVE; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t pk = __shfl_xor(key, j, WAVE);
      const uint32_t pl = __shfl_xor(lo, j, WAVE);
      const bool keep_min = (((lane & k) == 0) == ((lane & j) == 0));
      const bool mine_gt = (key > pk) || (key == pk && lo > pl);
      if (keep_min == mine_gt) { key = pk; lo = pl; }
    }
  }
}

}  // namespace verkv
