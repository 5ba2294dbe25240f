// PoissonComp (prefill) for gfx950: water-filling of the inclusion probabilities,
// the Poisson sample and the compaction of the pivotal set H u S.
//
// "Verify Before You Fetch" (picx.dev summary page, section "Methodology",
// subsection "POISSONCOMP"): r_i = min{1, c tau_i} with c such that
// sum_i min(1, c tau_i) = eta n (eq. 3); H are the tokens with r_i = 1, sink and
// local tokens among them; L the tokens with r_i < 1; S = {i in L : Z_i = 1} with
// independent Z_i ~ Bernoulli(r_i).
//
// Arithmetic (so that r and the sample are a deterministic function of the inputs):
// Q_i = ceil(tau_i 2^40) as an integer, exact 64-bit suffix sums S_m of Q over the
// non-forced tokens ranked by (Q descending, index ascending), water level
// c_m = fl(fl(B_rem - m) / fl(S_m)) with B_rem = fl(eta n) - |forced|, m* the first
// rank with B_rem - m > 0, S_m > 0 and fl(c_m Q_(m)) < 1, r = 1 on ranks < m* and
// fl(c_m* Q_i) after.  Z_i = [u_i < r_i], u_i the 53-bit Philox4x32-10 uniform of
// counter (i, kv_head, layer, sequence) and key (seed mod 2^32, seed >> 32).
//
// One workgroup of 1024 threads per (sequence, KV head).  Prefill work, not on the
// per-token decode path, so a single workgroup per head keeps the ranks exact
// without any cross-workgroup scan.
#include "kernels.h"

namespace verkv {

constexpr int PC_NT = 1024;
constexpr int PC_NW = PC_NT / WAVE;
constexpr int Q_BITS = 40;
constexpr int IDX_BITS = 20;                 // token index < 2^20 inside the sort key
constexpr uint64_t IDX_MASK = (1ull << IDX_BITS) - 1;

// Stable LSD radix sort of `n` 64-bit keys in src by their bits from `lo_bit` up (an
// even number of passes of 8 bits, `passes`); the result is back in `src`.  Keys that
// agree in those bits keep their input order.  One workgroup.  Within a tile of PC_NT
// keys the rank of a key among equal digits is found with wave ballots.
__device__ void block_radix_sort(uint64_t *src, uint64_t *dst, int n, int lo_bit, int passes,
                                 uint32_t *hist, uint32_t *wcnt /*[PC_NW][256]*/) {
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wv = tid / WAVE;
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = lo_bit + 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += PC_NT) atomicAdd(&hist[(src[i] >> shift) & 255], 1u);
    __syncthreads();
    if (tid == 0) {                       // exclusive scan of 256 digit counts
      uint32_t run = 0;
      for (int d = 0; d < 256; ++d) { uint32_t c = hist[d]; hist[d] = run; run += c; }
    }
    __syncthreads();
    for (int base = 0; base < n; base += PC_NT) {
      for (int j = tid; j < PC_NW * 256; j += PC_NT) wcnt[j] = 0;
      __syncthreads();
      const int i = base + tid;
      const bool valid = i < n;
      const uint64_t key = valid ? src[i] : 0ull;
      const uint32_t dig = (uint32_t)((key >> shift) & 255);
      uint64_t match = __ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const uint64_t b = __ballot(valid && ((dig >> bit) & 1));
        match &= ((dig >> bit) & 1) ? b : ~b;
      }
      const uint32_t rank = __popcll(match & lt_mask);
      // the highest lane of each equal-digit group publishes the group size
      if (valid && (match >> lane) == 1ull) wcnt[wv * 256 + dig] = __popcll(match);
      __syncthreads();
      if (tid < 256) {
        uint32_t run = hist[tid];
        for (int w = 0; w < PC_NW; ++w) {
          const uint32_t c = wcnt[w * 256 + tid];
          wcnt[w * 256 + tid] = run;
          run += c;
        }
        hist[tid] = run;
      }
      __syncthreads();
      if (valid) dst[wcnt[wv * 256 + dig] + rank] = key;
      __syncthreads();
    }
    uint64_t *tmp = src; src = dst; dst = tmp;
    __syncthreads();
  }
}

// Inclusive suffix sums of v over the workgroup's threads (thread t gets the sum over
// threads >= t), exact in 64-bit integers, and the workgroup's total.
__device__ uint64_t block_suffix_sum_u64(uint64_t v, uint64_t *wsum /*[PC_NW]*/, uint64_t *total) {
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wv = tid / WAVE;
  for (int off = 1; off < WAVE; off <<= 1) {
    const uint64_t o = __shfl_down(v, off, WAVE);
    if (lane + off < WAVE) v += o;
  }
  if (lane == 0) wsum[wv] = v;            // lane 0 holds its wave's total
  __syncthreads();
  uint64_t after = 0, tot = 0;
  for (int w = 0; w < PC_NW; ++w) {
    const uint64_t x = wsum[w];
    after += w > wv ? x : 0ull;
    tot += x;
  }
  __syncthreads();                        // wsum is reused by the next call
  *total = tot;
  return v + after;
}

constexpr int PC_SEL_CAP = 4096;             // keys the select path sorts in LDS (a power of 2)

// The water level from the M smallest keys alone (M = min(n_free, ceil(B_rem)) <= PC_SEL_CAP):
// m* must satisfy B_rem - m > 0, so it and every rank below it are among them.  An MSD
// radix select narrows a prefix of the 64-bit key until the keys at or below it (which
// hold the M smallest) fit in LDS; those are sorted there (bitonic), and
// S_m = (sum of Q over ranks m..M-1) + (total - sum over the M).  A token's rank is below
// m* exactly when its key is below the key of rank m* (keys are distinct).  Same r, level
// and arithmetic as sorting all keys.
__device__ void poissoncomp_select(const CompressArgs &a, int unit, const uint64_t *ka, uint64_t *kb,
                                   double *r, int nfree, int M, double b_rem, int64_t total,
                                   uint32_t *hist, int64_t *isum, uint64_t *wsum, uint64_t *s_col,
                                   int32_t *s_sel) {
  const int tid = threadIdx.x;
  auto q_of = [](uint64_t k) -> uint64_t { return (1ull << Q_BITS) - (k >> IDX_BITS); };
  // narrow the prefix: keys k with (k >> sh) <= pre are collected (sh = 64: all keys)
  uint64_t pre = 0;
  int sh = 64;
  int64_t kk = M;                          // rank of the M-th smallest key among those at pre
  int64_t match = nfree;                   // keys whose bits above sh equal pre
  while ((int64_t)M - kk + match > PC_SEL_CAP) {
    const int ns = sh - 8;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < nfree; j += PC_NT) {
      const uint64_t k = ka[j];
      if (sh == 64 || (k >> sh) == pre) atomicAdd(&hist[(k >> ns) & 255], 1u);
    }
    __syncthreads();
    if (tid == 0) {                        // the bucket holding the kk-th of them
      int b = 0;
      int64_t left = kk;
      while (b < 255 && left > (int64_t)hist[b]) { left -= hist[b]; ++b; }
      s_sel[0] = b;
      s_sel[1] = (int32_t)left;
      s_sel[2] = (int32_t)hist[b];
    }
    __syncthreads();
    pre = (sh == 64 ? 0ull : (pre << 8)) | (uint64_t)s_sel[0];
    kk = s_sel[1];
    match = s_sel[2];
    sh = ns;
    __syncthreads();                       // s_sel is rewritten by the next pass
  }
  // collect, pad to a power of two, sort ascending
  if (tid == 0) s_sel[0] = 0;
  __syncthreads();
  for (int j = tid; j < nfree; j += PC_NT) {
    const uint64_t k = ka[j];
    if (sh == 64 || (k >> sh) <= pre) {
      const int at = atomicAdd(&s_sel[0], 1);
      if (at < PC_SEL_CAP) s_col[at] = k;
    }
  }
  __syncthreads();
  const int ncol = min(s_sel[0], PC_SEL_CAP);
  int p2 = 1;
  while (p2 < ncol) p2 <<= 1;
  for (int i = ncol + tid; i < p2; i += PC_NT) s_col[i] = ~0ull;
  __syncthreads();
  for (int k2 = 2; k2 <= p2; k2 <<= 1) {
    for (int j2 = k2 >> 1; j2 > 0; j2 >>= 1) {
      for (int i = tid; i < p2; i += PC_NT) {
        const int l = i ^ j2;
        if (l > i) {
          const uint64_t x = s_col[i], y = s_col[l];
          if ((x > y) == ((i & k2) == 0)) {
            s_col[i] = y;
            s_col[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  // S_m for the M ranks -> kb[m]
  int64_t part = 0;
  for (int m = tid; m < M; m += PC_NT) part += (int64_t)q_of(s_col[m]);
  const int64_t sum_m = block_sum_i64<PC_NT>(part, isum);
  uint64_t carry = (uint64_t)(total - sum_m);
  for (int tix = (M + PC_NT - 1) / PC_NT - 1; tix >= 0; --tix) {
    const int m = tix * PC_NT + tid;
    const uint64_t q = m < M ? q_of(s_col[m]) : 0ull;
    uint64_t tile = 0;
    const uint64_t sfx = block_suffix_sum_u64(q, wsum, &tile);
    if (m < M) kb[m] = sfx + carry;
    carry += tile;
  }
  // m*: smallest rank whose water level leaves it unsaturated
  if (tid == 0) s_sel[0] = INT32_MAX;
  __syncthreads();
  for (int m = tid; m < M; m += PC_NT) {
    const double rem = b_rem - (double)m;
    const uint64_t sm = kb[m];
    if (rem > 0.0 && sm > 0) {
      const double c = rem / (double)sm;
      if (c * (double)q_of(s_col[m]) < 1.0) atomicMin(&s_sel[0], m);
    }
  }
  __syncthreads();
  const int mstar = s_sel[0];
  if (a.level && tid == 0)
    a.level[unit] = mstar == INT32_MAX ? LEVEL_SATURATED : (b_rem - (double)mstar) / (double)kb[mstar];
  if (mstar == INT32_MAX) {                // every positive score saturates
    for (int j = tid; j < nfree; j += PC_NT) {
      const uint64_t k = ka[j];
      r[(int)(k & IDX_MASK)] = q_of(k) > 0 ? 1.0 : 0.0;
    }
  } else {
    const double c = (b_rem - (double)mstar) / (double)kb[mstar];
    const uint64_t th = s_col[mstar];
    for (int j = tid; j < nfree; j += PC_NT) {
      const uint64_t k = ka[j];
      r[(int)(k & IDX_MASK)] = k < th ? 1.0 : c * (double)q_of(k);
    }
  }
}

__global__ __launch_bounds__(PC_NT) void k_poissoncomp(CompressArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wcnt[PC_NW * 256];
  __shared__ uint64_t wsum[PC_NW];
  __shared__ int64_t isum[PC_NW];
  __shared__ uint64_t s_col[PC_SEL_CAP];
  __shared__ int32_t s_sel[3];
  __shared__ int32_t iscratch[PC_NW];
  __shared__ int32_t s_mstar;

  const int unit = blockIdx.x;
  const int b = unit / a.t.Hkv;
  const int g = unit % a.t.Hkv;
  const int n = a.t.s[b].n;
  const int tid = threadIdx.x;
  const int64_t tb = tok_base(a.t, b, g);
  const float *tau = a.tau + tb;
  double *r = a.r + tb;
  uint64_t *ka = a.keys_a + tb;
  uint64_t *kb = a.keys_b + tb;

  // forced tokens: [0, lo) and [hi, n)
  const int lo = min(a.t.n_sink, n);
  const int hi = max(lo, n - a.t.n_local);
  const int nfree = hi - lo;
  const double b_rem = a.eta * (double)n - (double)(n - nfree);

  // tau range check and forced tokens
  for (int i = tid; i < n; i += PC_NT) {
    const float x = tau[i];
    if (!(x >= 0.0f && x <= 1.0f)) atomicOr(&a.status[0], 1);
    if (i < lo || i >= hi) r[i] = 1.0;
  }

  if (nfree > 0 && b_rem > 0.0 && b_rem < (double)nfree) {
    // sort keys: (2^40 - Q) << 20 | index  ->  ascending = Q descending, index ascending,
    // and the exact total of Q
    int64_t qsum = 0;
    for (int j = tid; j < nfree; j += PC_NT) {
      const int i = lo + j;
      const float x = tau[i];
      const double xs = (double)(x > 0.0f ? x : 0.0f) * 0x1.0p40;
      const uint64_t q = (uint64_t)ceil(xs);
      ka[j] = (((1ull << Q_BITS) - q) << IDX_BITS) | (uint64_t)i;
      qsum += (int64_t)q;
    }
    const int64_t total = block_sum_i64<PC_NT>(qsum, isum);   // its barriers publish ka
    // m* needs B_rem - m > 0, so only the M smallest keys can be ranks below it or m*
    const int M = (int)fmin((double)nfree, ceil(b_rem));
    if (M <= PC_SEL_CAP) {
      poissoncomp_select(a, unit, ka, kb, r, nfree, M, b_rem, total, hist, isum, wsum, s_col, s_sel);
    } else {
    // They are written in index order and the sort is stable, so sorting by bits 20-60
    // (2^40 - Q < 2^41) alone gives the order of the whole keys: six passes, not eight.
    static_assert(IDX_BITS + Q_BITS + 1 <= IDX_BITS + 8 * 6, "six passes cover 2^40 - Q");
    block_radix_sort(ka, kb, nfree, IDX_BITS, 6, hist, wcnt);

    // exact suffix sums S_m of Q over ranks, tile by tile from the end -> kb[m]
    uint64_t carry = 0;
    const int ntile = (nfree + PC_NT - 1) / PC_NT;
    for (int tix = ntile - 1; tix >= 0; --tix) {
      const int m = tix * PC_NT + tid;
      const uint64_t q = (m < nfree) ? ((1ull << Q_BITS) - (ka[m] >> IDX_BITS)) : 0ull;
      uint64_t tile = 0;
      const uint64_t sfx = block_suffix_sum_u64(q, wsum, &tile);
      if (m < nfree) kb[m] = sfx + carry;
      carry += tile;
    }

    // m*: smallest rank whose water level leaves it unsaturated
    if (tid == 0) s_mstar = INT32_MAX;
    __syncthreads();
    for (int m = tid; m < nfree; m += PC_NT) {
      const double rem = b_rem - (double)m;
      const uint64_t s = kb[m];
      if (rem > 0.0 && s > 0) {
        const double c = rem / (double)s;
        const uint64_t q = (1ull << Q_BITS) - (ka[m] >> IDX_BITS);
        if (c * (double)q < 1.0) atomicMin(&s_mstar, m);
      }
    }
    __syncthreads();
    const int mstar = s_mstar;
    if (a.level && tid == 0)
      a.level[unit] = mstar == INT32_MAX ? LEVEL_SATURATED
                                         : (b_rem - (double)mstar) / (double)kb[mstar];
    if (mstar == INT32_MAX) {
      // every positive score saturates; the budget cannot be spent
      for (int m = tid; m < nfree; m += PC_NT) {
        const uint64_t q = (1ull << Q_BITS) - (ka[m] >> IDX_BITS);
        r[(int)(ka[m] & IDX_MASK)] = q > 0 ? 1.0 : 0.0;
      }
    } else {
      const double c = (b_rem - (double)mstar) / (double)kb[mstar];
      for (int m = tid; m < nfree; m += PC_NT) {
        const uint64_t q = (1ull << Q_BITS) - (ka[m] >> IDX_BITS);
        r[(int)(ka[m] & IDX_MASK)] = (m < mstar) ? 1.0 : c * (double)q;
      }
    }
    }
  } else {
    const double v = (nfree > 0 && b_rem >= (double)nfree) ? 1.0 : 0.0;
    for (int i = lo + tid; i < hi; i += PC_NT) r[i] = v;
    if (a.level && tid == 0)
      a.level[unit] = (nfree == 0 || b_rem >= (double)nfree) ? LEVEL_ALL : LEVEL_NONE;
  }
  __syncthreads();

  // Poisson draw and the resident mask, then ascending compaction of H u S.
  const int W = words_of(n);
  const int wpt = (W + PC_NT - 1) / PC_NT;           // contiguous words per thread
  const int w0 = tid * wpt;
  const int w1 = min(W, w0 + wpt);
  uint32_t *res = a.resident + word_base(a.t, b, g);
  int32_t cnt = 0;
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = 0;
    for (int j = 0; j < 32; ++j) {
      const int i = 32 * w + j;
      if (i >= n) break;
      const double ri = r[i];
      bool keep = ri >= 1.0;
      if (!keep && ri > 0.0)
        keep = philox_uniform53((uint32_t)i, (uint32_t)g, a.layer, (uint32_t)b, a.seed) < ri;
      bits |= (uint32_t)keep << j;
    }
    res[w] = bits;
    cnt += __popc(bits);
  }
  // words past the sequence's length (capacity for appended tokens) start empty
  for (int w = W + tid; w < words_of(a.t.s[b].cap); w += PC_NT) res[w] = 0u;
  int32_t total;
  int32_t pos = block_excl_scan<PC_NT>(cnt, iscratch, &total);
  int32_t *pidx = a.piv_idx + (int64_t)unit * a.cap;
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = res[w];
    while (bits) {
      const int j = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < a.cap) pidx[pos] = 32 * w + j;
      ++pos;
    }
  }
  if (tid == 0) {
    a.piv_count[unit] = total;
    atomicMax(&a.status[1], total);
  }
}

// Copy the K/V rows of the pivots from the pinned host cache (zero-copy reads) to the
// places the pivot-attention schedule reads them from (pivot_store_row).
__global__ __launch_bounds__(256) void k_gather_pivots(GatherArgs a) {
  const int unit = blockIdx.y;
  const int b = unit / a.t.Hkv;
  const int g = unit % a.t.Hkv;
  const int cnt = min(a.piv_count[unit], a.cap);
  const int p0 = blockIdx.x * GATHER_ROWS;
  // rows [cnt, whole chunks) of the head's last chunk are written as zeros: the pivot
  // attention may load them (with weight 0) before it knows where the head ends
  const int cntp = (cnt + PIVOT_CHUNK - 1) / PIVOT_CHUNK * PIVOT_CHUNK;
  if (p0 >= cntp) return;
  const int4 hdr = a.sched[2 * a.workers];
  const int64_t NC = hdr.x, P = hdr.y;
  if (NC <= 0 || P <= 0) return;
  const int64_t c_u = a.runs[unit].z;
  const int per_row = a.row_bytes / 16;                // 16-byte pieces per row
  const int64_t src_row0 = tok_base(a.t, b, g);
  const int nrow = min(GATHER_ROWS, cntp - p0);
  for (int e = threadIdx.x; e < nrow * per_row; e += blockDim.x) {
    const int p = p0 + e / per_row;
    const int piece = e % per_row;
    const int64_t row = pivot_store_row(c_u, p, NC, P);
    if (row < 0 || row >= a.rows) continue;            // never, for a schedule of these counts
    const int64_t dof = row * a.row_bytes + (int64_t)piece * 16;
    uint4 kk = make_uint4(0u, 0u, 0u, 0u), vv = kk;
    if (p < cnt) {
      const int64_t tok = a.piv_idx[(int64_t)unit * a.cap + p];
      const int64_t so = (src_row0 + tok) * a.row_bytes + (int64_t)piece * 16;
      kk = *(const uint4 *)(a.K_host + so);
      vv = *(const uint4 *)(a.V_host + so);
    }
    *(uint4 *)(a.piv_k + dof) = kk;
    *(uint4 *)(a.piv_v + dof) = vv;
  }
}

hipError_t launch_poissoncomp(const CompressArgs &a, int units, hipStream_t st) {
  return launch_kernel(k_poissoncomp, dim3(units), dim3(PC_NT), 0, st, a);
}

hipError_t launch_gather_pivots(const GatherArgs &a, int units, hipStream_t st) {
  const int nblk = (a.cap + GATHER_ROWS - 1) / GATHER_ROWS;
  return launch_kernel(k_gather_pivots, dim3(nblk, units), dim3(256), 0, st, a);
}

}  // namespace verkv
