// KVFetch step 1 for gfx950: sketch scores of every cached token for every query
// row of a KV head, in float64 ("Verify Before You Fetch", picx.dev summary page,
// "KVFETCH" step 1: estimated weights w_hat_i from the sketch; the decisions of
// steps 2-4 are made on these weights, so they are kept in float64 end to end).
//
// Streaming layout: a workgroup (256 threads for bf16, 512 for float32 rows) owns
// SKETCH_CHUNK = 256 tokens of one
// (sequence, KV head).  Each lane loads one 16-byte slice of a key row (8 bf16 or 4
// float32 elements), so a wave instruction reads 1 KB of contiguous rows; the G query
// rows stay in registers as float64 and the per-lane partial dot products are summed
// across the lanes of a row with DPP butterflies.  The chunk keeps its scores in
// registers, takes the per-row chunk maximum m_c, and writes
//   wc_i = exp(s_i - m_c)       (float64, [row][token])
//   (m_c, sum_i wc_i)           per (row, chunk)
// The decision kernel rescales by exp(m_c - m_hat) once m_hat = max_c m_c is known.
// The same workgroup clears the chunk's words of the step's fetch bitmask.
#include "kernels.h"

namespace verkv {

// bf16 rows: 4 waves of 64 tokens; float32 rows (32 lanes per row): 8 waves of 32
// tokens, so that every lane keeps 16 scores either way.
template <bool BF16>
struct SketchCfg {
  static constexpr int NT = BF16 ? 256 : 512;
  static constexpr int NW = NT / WAVE;
};

// Map a flat block index to (sequence, KV head, chunk).
__device__ __forceinline__ void sketch_block(const SeqTable &t, int blk, int &b, int &g, int &c) {
  int lo = 0, hi = t.B - 1;
  while (lo < hi) {                       // last sequence whose first block <= blk
    const int mid = (lo + hi + 1) >> 1;
    if (t.Hkv * t.s[mid].chunk_off <= blk) lo = mid; else hi = mid - 1;
  }
  b = lo;
  const int rel = blk - t.Hkv * t.s[b].chunk_off;
  const int nch = chunks_of(t.s[b].n);
  g = rel / nch;
  c = rel % nch;
}

template <bool BF16, int G>
__global__ __launch_bounds__(SketchCfg<BF16>::NT) void k_sketch(SketchArgs a) {
  constexpr int SK_NW = SketchCfg<BF16>::NW;
  using RS = RowSlice<BF16>;
  constexpr int EPL = RS::EPL;              // elements per lane
  constexpr int LPT = D / EPL;              // lanes per token row (16 or 32)
  constexpr int TPW = WAVE / LPT;           // token rows per wave instruction (4 or 2)
  constexpr int TOK_PER_WAVE = SKETCH_CHUNK / SK_NW;
  constexpr int ITER = TOK_PER_WAVE / TPW;  // 16
  constexpr int BATCH = 8;                  // loads in flight per lane
  constexpr int ROW_BYTES = D * (BF16 ? 2 : 4);

  __shared__ double s_red[SK_NW][G];
  __shared__ double s_f0[SK_NW][G];

  int b, g, c;
  sketch_block(a.t, blockIdx.x, b, g, c);
  const int n = a.t.s[b].n;
  const int Hq = a.t.Hkv * G;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wv = threadIdx.x / WAVE;
  const int sub = lane % LPT;               // slice of the row this lane owns
  const int grp = lane / LPT;               // which of the TPW rows of an instruction
  const int d0 = sub * EPL;

  // clear this chunk's words of the fetch bitmask (SKETCH_CHUNK / 32 words), and on
  // chunk 0 the per-row counters of the decision kernel for the G rows of this head
  if (threadIdx.x < SKETCH_CHUNK / 32) {
    const int w = c * (SKETCH_CHUNK / 32) + threadIdx.x;
    if (w < words_of(n)) a.fbits[word_base(a.t, b, g) + w] = 0u;
  }
  if (c == 0 && threadIdx.x < G) {
    const int64_t row = (int64_t)b * a.t.Hkv * G + g * G + threadIdx.x;
    a.bar[row] = 0u;
    a.wcount[row] = 0u;
    a.kstar[row] = 0;
  }

  // query slices in float64
  double qd[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float *qr = a.q + ((int64_t)b * Hq + g * G + j) * D + d0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qd[j][e] = (double)qr[e];
  }

  const int tok0 = c * SKETCH_CHUNK + wv * TOK_PER_WAVE;
  const uint8_t *rows = a.sketch + tok_base(a.t, b, g) * ROW_BYTES;
  const int myrow = sub < G ? sub : 0;      // the query row whose scores this lane keeps
  double keep[ITER];

#pragma unroll
  for (int it0 = 0; it0 < ITER; it0 += BATCH) {
    uint4 raw[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int tok = tok0 + (it0 + k) * TPW + grp;
      raw[k] = tok < n ? *(const uint4 *)(rows + (int64_t)tok * ROW_BYTES + d0 * (BF16 ? 2 : 4))
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      float x[EPL];
      RS::widen(raw[k], x);
      double acc[G];
#pragma unroll
      for (int j = 0; j < G; ++j) acc[j] = 0.0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const double xe = (double)x[e];
#pragma unroll
        for (int j = 0; j < G; ++j) acc[j] = fma(qd[j][e], xe, acc[j]);
      }
      double mine = 0.0;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        double v = sum16(acc[j]);
        if (LPT == 32) v += shfl_xor_d(v, 16);
        mine = (j == myrow) ? v : mine;
      }
      const int tok = tok0 + (it0 + k) * TPW + grp;
      keep[it0 + k] = tok < n ? mine / a.sqrt_d : -INFINITY;
    }
  }

  // per-row chunk maximum: lanes with the same `sub` hold the same row
  double mx = -INFINITY;
#pragma unroll
  for (int it = 0; it < ITER; ++it) mx = fmax(mx, keep[it]);
  for (int m = LPT; m < WAVE; m <<= 1) mx = fmax(mx, shfl_xor_d(mx, m));
  if (grp == 0 && sub < G) s_red[wv][sub] = mx;
  __syncthreads();
  double mc = s_red[0][myrow];
#pragma unroll
  for (int w = 1; w < SK_NW; ++w) mc = fmax(mc, s_red[w][myrow]);
  __syncthreads();

  // exp(s - m_c), their sum D_c, and f(0)_c = sum over L of exp(s - m_c)(1 - r): the
  // bias of the shrinkage estimator at beta = 0, where every lambda_i equals r_i
  double sum = 0.0, f0 = 0.0;
  double *wrow = a.wc + row_tok_base(a.t, b, g * G + myrow);
  const double *rr = a.r + tok_base(a.t, b, g);
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int tok = tok0 + it * TPW + grp;
    const double e = exp(keep[it] - mc);
    const double ri = tok < n ? rr[tok] : 1.0;
    sum += e;
    if (ri < 1.0) f0 += e * (1.0 - ri);
    if (sub < G && tok < n) wrow[tok] = e;
  }
  for (int m = LPT; m < WAVE; m <<= 1) {
    sum += shfl_xor_d(sum, m);
    f0 += shfl_xor_d(f0, m);
  }
  if (grp == 0 && sub < G) { s_red[wv][sub] = sum; s_f0[wv][sub] = f0; }
  __syncthreads();
  if (threadIdx.x < G) {
    double s = 0.0, z = 0.0;
#pragma unroll
    for (int w = 0; w < SK_NW; ++w) { s += s_red[w][threadIdx.x]; z += s_f0[w][threadIdx.x]; }
    // thread j is lane j of wave 0, whose `sub` is j, so `mc` is row j's maximum
    const int64_t o = row_chunk_base(a.t, b, g * G + threadIdx.x) + c;
    a.cstat[o] = make_double2(mc, s);
    a.cf0[o] = z;
  }
}

template <bool BF16, int G>
static hipError_t launch_sketch_t(const SketchArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((k_sketch<BF16, G>), dim3(a.total_blocks), dim3(SketchCfg<BF16>::NT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_sketch(const SketchArgs &a, bool bf16, hipStream_t st) {
  switch (a.t.G * 2 + (bf16 ? 1 : 0)) {
#define VERKV_SK_CASE(GG)                                        \
  case GG * 2 + 1: return launch_sketch_t<true, GG>(a, st);      \
  case GG * 2: return launch_sketch_t<false, GG>(a, st);
    VERKV_SK_CASE(1) VERKV_SK_CASE(2) VERKV_SK_CASE(3) VERKV_SK_CASE(4)
    VERKV_SK_CASE(5) VERKV_SK_CASE(6) VERKV_SK_CASE(7) VERKV_SK_CASE(8)
#undef VERKV_SK_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace verkv
