// KVFetch step 1 for gfx950: sketch scores of every cached token for every query
// row of a KV head, in float64 ("Verify Before You Fetch", picx.dev summary page,
// "KVFETCH" step 1: estimated weights w_hat_i from the sketch; the decisions of
// steps 2-4 are made on these weights, so they are kept in float64 end to end).
//
// Streaming layout: one wave owns SKETCH_CHUNK = 128 tokens of one (sequence, KV
// head).  A key row is split over 8 lanes (16 when the group has more than four query
// rows), each holding its float64 query elements in registers, so one wave load reads
// whole rows (1 KB contiguous).  The per-lane partial dot products of four query rows
// are reduce-scattered over the row's lanes with DPP exchanges (four exchanges over 8
// lanes instead of three butterfly levels per query row).  Scores wait in LDS for the
// per-row chunk maximum m_c; the wave writes
//   wc_i = exp(s_i - m_c)            (float64, [row][token], whole lines)
//   (m_c, sum_i wc_i), f(0)_c        per (row, chunk)
// where f(0)_c = sum over the chunk's tokens of L of wc_i (1 - r_i): the bias of the
// shrinkage estimator at beta = 0.  The decision kernel rescales by exp(m_c - m_hat)
// once m_hat = max_c m_c is known.  The workgroup also clears the chunk's words of the
// step's fetch bitmask and, on chunk 0, the decision kernel's per-row counters and
// exchange sequence words.
//
// With a 2-bit sketch (Q2) a row is 64 bytes of codes and group parameters (the layout
// k_quant_sketch writes); a lane reads the code word and the (mn, sc) pairs of its two
// 8-dimension pieces and forms x_hat = mn + code * sc in float64 before the same dot
// products, so the sketch keys are bit-identical to the quantiser's definition.
#include "kernels.h"

namespace verkv {

constexpr int SK_WAVES = 4;               // waves per workgroup, one chunk each

// Map a flat chunk index (over the chunks of every head's capacity) to (sequence, KV
// head, chunk); chunks past a head's length get c >= chunks_of(n) and do nothing.
__device__ __forceinline__ void sketch_chunk(const SeqTable &t, int blk, int &b, int &g, int &c) {
  int lo = 0, hi = t.B - 1;
  while (lo < hi) {                       // last sequence whose first chunk <= blk
    const int mid = (lo + hi + 1) >> 1;
    if (t.Hkv * t.s[mid].chunk_off <= blk) lo = mid; else hi = mid - 1;
  }
  b = lo;
  const int rel = blk - t.Hkv * t.s[b].chunk_off;
  const int nch = chunks_of(t.s[b].cap);
  g = rel / nch;
  c = rel % nch;
}

// Reduce-scatters of four per-lane partials v[0..3] over the lanes that share a token.
// 16 lanes (one DPP row): on return lanes 4r..4r+3 of the row hold the total of v[r].
__device__ __forceinline__ double reduce_scatter4x16(const double *v, int s) {
  const bool b3 = (s >> 3) & 1;
  const bool b2 = (s >> 2) & 1;
  // lanes i and i^8: bit 3 clear keeps {0,1}, set keeps {2,3}
  double k0 = b3 ? v[2] : v[0], k1 = b3 ? v[3] : v[1];
  const double s0 = b3 ? v[0] : v[2], s1 = b3 ? v[1] : v[3];
  k0 += dpp_d<DPP_ROR8>(s0);
  k1 += dpp_d<DPP_ROR8>(s1);
  // lanes i and 7-i of each half row: bit 2 clear keeps the first, set the second
  double k = b2 ? k1 : k0;
  const double o = b2 ? k0 : k1;
  k += dpp_d<DPP_HALF_MIRROR>(o);
  // the four lanes of the quad now cover all 16 lanes between them
  k += dpp_d<DPP_XOR1>(k);
  k += dpp_d<DPP_XOR2>(k);
  return k;
}
// 8 lanes (half a DPP row): on return lanes 2r, 2r+1 of the group hold the total of v[r].
__device__ __forceinline__ double reduce_scatter4x8(const double *v, int s) {
  const bool b2 = (s >> 2) & 1;
  const bool b1 = (s >> 1) & 1;
  // lanes i and 7-i: lanes 0-3 keep {0,1}, lanes 4-7 keep {2,3}
  double k0 = b2 ? v[2] : v[0], k1 = b2 ? v[3] : v[1];
  const double s0 = b2 ? v[0] : v[2], s1 = b2 ? v[1] : v[3];
  k0 += dpp_d<DPP_HALF_MIRROR>(s0);
  k1 += dpp_d<DPP_HALF_MIRROR>(s1);
  // lanes i and i^2: bit 1 clear keeps the first, set the second
  double k = b1 ? k1 : k0;
  const double o = b1 ? k0 : k1;
  k += dpp_d<DPP_XOR2>(o);
  k += dpp_d<DPP_XOR1>(k);
  return k;
}

// One wave streams one chunk of SKETCH_CHUNK tokens.  A token row is split over LPT
// lanes (8 when G <= 4, else 16, so the float64 query slices of the G rows fit in
// registers); a load step reads 64 / LPT whole rows with one or more fully used 1 KB
// wave loads, and batches of 8 loads per lane are kept one batch ahead of the
// arithmetic.  Scores wait in the wave's own LDS region for the chunk maximum; then
// each lane takes CH / 64 tokens of every row for exp, the sums and the stores.  Waves
// never wait for each other.
template <bool BF16, int G, bool Q2 = false>
__global__ __launch_bounds__(SK_WAVES * WAVE) void k_sketch(SketchArgs a) {
  using RS = RowSlice<BF16 || Q2>;          // Q2: pieces of 8 dimensions, as bf16 rows
  constexpr int CH = SKETCH_CHUNK;
  constexpr int EPP = RS::EPL;              // elements per 16-byte piece
  constexpr int LPT = G <= 4 ? 8 : 16;      // lanes per token row
  constexpr int TPS = WAVE / LPT;           // tokens per load step
  constexpr int ROW_BYTES = Q2 ? SKETCH2_ROW_BYTES : D * (BF16 ? 2 : 4);
  constexpr int PPL = D * ((BF16 || Q2) ? 2 : 4) / 16 / LPT;   // pieces per lane per token
  constexpr int EPT = PPL * EPP;            // elements per lane per token
  constexpr int STEPS = CH / TPS;
  constexpr int SB = 8 / PPL;               // load steps per batch
  constexpr int NB = STEPS / SB;
  constexpr int NG4 = (G + 3) / 4;          // groups of four query rows
  constexpr int TPL = CH / WAVE;            // tokens per lane in the exp phase
  static_assert(PPL >= 1 && STEPS % SB == 0 && CH % WAVE == 0, "sketch tiling");

  __shared__ double s_sc[SK_WAVES][G][CH];

  const int lane = threadIdx.x & (WAVE - 1);
  const int wv = threadIdx.x / WAVE;
  const int flat = blockIdx.x * SK_WAVES + wv;
  if (flat >= a.total_blocks) return;       // whole wave; no block barriers below
  int b, g, c;
  sketch_chunk(a.t, flat, b, g, c);
  const int n = a.t.s[b].n;
  if (c >= chunks_of(n)) return;            // capacity beyond the sequence's length
  const int Hq = a.t.Hkv * G;
  const int sidx = lane & (LPT - 1);        // lane within the token's group
  const int tsub = lane / LPT;              // token of the load step
  // G = 4 over 8 lanes: lane s keeps query row (slot ^ pm) in register slot `slot`, with
  // pm = 0, 0, 1, 1, 3, 3, 2, 2 for s = 0..7, so every level of the reduce-scatter keeps
  // and sends the same slots in every lane (no per-lane selects); it ends with row pm.
  constexpr bool PERM = (G == 4 && LPT == 8);
  const int pm = (((sidx >> 2) & 1) << 1) | (((sidx >> 1) ^ (sidx >> 2)) & 1);
  const int rsel = PERM ? pm : (LPT == 8 ? (sidx >> 1) & 3 : (sidx >> 2) & 3);   // row it ends with
  const bool writer = LPT == 8 ? (sidx & 1) == 0 : (sidx & 3) == 0;
  const int base = c * CH;
  double (*sc)[CH] = s_sc[wv];

  // clear this chunk's words of the fetch bitmask, and on chunk 0 the per-row counters
  // of the decision kernel for the G rows of this head
  if (lane < CH / 32) {
    const int w = c * (CH / 32) + lane;
    if (w < words_of(n)) a.fbits[word_base(a.t, b, g) + w] = 0u;
  }
  if (c == 0) {
    const int64_t row0 = ((int64_t)b * a.t.Hkv + g) * G;
    if (lane < G) {
      a.wcount[row0 + lane] = 0u;
      a.kstar[row0 + lane] = 0;
    }
    for (int i = lane; i < G * a.xseq_row; i += WAVE) a.xseq[row0 * a.xseq_row + i] = 0.0;
  }

  // float64 query elements of the pieces sidx, sidx + LPT, ...
  double qd[G][EPT];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int jr = PERM ? (j ^ pm) : j;       // the query row of register slot j
    const float *qr = a.q + ((int64_t)b * Hq + g * G + jr) * D;
#pragma unroll
    for (int p = 0; p < PPL; ++p)
#pragma unroll
      for (int e = 0; e < EPP; ++e) qd[j][p * EPP + e] = (double)qr[(sidx + p * LPT) * EPP + e];
  }

  // rows past n (the last chunk) re-read row n-1; their scores are replaced by -inf
  const uint8_t *rows = a.sketch + tok_base(a.t, b, g) * ROW_BYTES + (Q2 ? 0 : sidx * 16);
  auto load_batch = [&](int bi, uint4 *raw) {
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      const int tok = min(base + (bi * SB + k) * TPS + tsub, n - 1);
      const uint8_t *rp = rows + (int64_t)tok * ROW_BYTES;
      if constexpr (Q2) {
        // .x: the code word of pieces (sidx & 7) and (sidx & 7) + 8; .y-.w: parameters.
        // LPT 8: pieces sidx, sidx + 8 -> (mn, sc) of groups sidx/4 and sidx/4 + 2, one
        // 16-byte read; LPT 16: piece sidx -> (mn, sc) of group sidx/4
        uint4 r;
        r.x = *(const uint32_t *)(rp + 4 * (sidx & 7));
        if constexpr (LPT == 8) {
          const uint4 pm = *(const uint4 *)(rp + 32 + 16 * ((sidx >> 2) & 1));
          raw[2 * k] = make_uint4(r.x, pm.x, pm.y, 0u);
          raw[2 * k + 1] = make_uint4(r.x >> 16, pm.z, pm.w, 0u);
        } else {
          const int gq = sidx >> 2;
          const uint2 pm = *(const uint2 *)(rp + 32 + 4 * ((gq & 1) * 4 + (gq >> 1) * 2));
          raw[k] = make_uint4(r.x >> (16 * (sidx >> 3)), pm.x, pm.y, 0u);
        }
      } else {
#pragma unroll
        for (int p = 0; p < PPL; ++p) raw[k * PPL + p] = load_stream16(rp + p * LPT * 16);
      }
    }
  };
  // two batch buffers alternate; the batch loop is unrolled so each buffer keeps its
  // registers (a copy from the buffer in flight would wait for its loads)
  uint4 bufA[SB * PPL], bufB[SB * PPL];
  double run_max = -INFINITY;               // max of this lane's scores of row rsel
  auto compute = [&](int bi, const uint4 *cur) {
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      double acc[NG4 * 4];
#pragma unroll
      for (int j = 0; j < NG4 * 4; ++j) acc[j] = 0.0;
#pragma unroll
      for (int p = 0; p < PPL; ++p) {
        if constexpr (Q2) {
          // piece codes in bits 0-15 of .x, (mn, sc) in .y, .z
          const uint4 r = cur[k * PPL + p];
          const double mn = (double)__uint_as_float(r.y), scl = (double)__uint_as_float(r.z);
#pragma unroll
          for (int e = 0; e < EPP; ++e) {
            const double xe = fma((double)((r.x >> (2 * e)) & 3u), scl, mn);
#pragma unroll
            for (int j = 0; j < G; ++j) acc[j] = fma(qd[j][p * EPP + e], xe, acc[j]);
          }
        } else {
          float x[EPP];
          RS::widen(cur[k * PPL + p], x);
#pragma unroll
          for (int e = 0; e < EPP; ++e) {
            const double xe = (double)x[e];
#pragma unroll
            for (int j = 0; j < G; ++j) acc[j] = fma(qd[j][p * EPP + e], xe, acc[j]);
          }
        }
      }
      const int tk = (bi * SB + k) * TPS + tsub;        // token within the chunk
#pragma unroll
      for (int q4 = 0; q4 < NG4; ++q4) {
        double v;
        if constexpr (PERM) {
          // lanes i and 7-i: keep slots 0, 1 and add the partner's slots 2, 3 (its rows
          // 0, 1 here); lanes i and i^2: keep slot 0, add the partner's slot 1; then the
          // pair i, i^1 holds the same row
          double k0 = acc[0] + dpp_d<DPP_HALF_MIRROR>(acc[2]);
          const double k1 = acc[1] + dpp_d<DPP_HALF_MIRROR>(acc[3]);
          k0 += dpp_d<DPP_XOR2>(k1);
          v = k0 + dpp_d<DPP_XOR1>(k0);
        } else {
          v = LPT == 8 ? reduce_scatter4x8(acc + 4 * q4, sidx)
                       : reduce_scatter4x16(acc + 4 * q4, sidx);
        }
        const int j = 4 * q4 + rsel;
        const double sv = base + tk < n ? v * a.inv_sqrt_d : -INFINITY;
        if (writer && j < G) sc[j][tk] = sv;
        if (NG4 == 1) run_max = fmax(run_max, sv);
      }
    }
  };
  load_batch(0, bufA);
#pragma unroll
  for (int bi = 0; bi < NB; ++bi) {
    if (bi + 1 < NB) load_batch(bi + 1, (bi & 1) ? bufA : bufB);
    compute(bi, (bi & 1) ? bufB : bufA);
  }
  __builtin_amdgcn_wave_barrier();

  // chunk maxima m_c of the G rows, wave-uniform
  double mrow[G];
  if (NG4 == 1) {
    // lanes with equal rsel differ in bit 0 and bits 3-5 (LPT 8)
    double m = run_max;
    m = fmax(m, dpp_d<DPP_XOR1>(m));
    m = fmax(m, dpp_d<DPP_ROR8>(m));
    m = fmax(m, shfl_xor_d(m, 16));
    m = fmax(m, shfl_xor_d(m, 32));
#pragma unroll
    for (int j = 0; j < G; ++j) {
      // the lane that ends with row j: 2 j, or 0, 2, 6, 4 for the permuted slots
      const int lj = PERM ? (j == 0 ? 0 : j == 1 ? 2 : j == 2 ? 6 : 4) : 2 * j;
      mrow[j] = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(m), lj),
                                 __builtin_amdgcn_readlane(__double2loint(m), lj));
    }
  } else {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      double m = -INFINITY;
#pragma unroll
      for (int u = 0; u < TPL; ++u) m = fmax(m, sc[j][lane + u * WAVE]);
      m = max16(m);
      m = fmax(m, shfl_xor_d(m, 16));
      mrow[j] = fmax(m, shfl_xor_d(m, 32));
    }
  }

  // wc = exp(s - m_c), D_c = sum of wc, f(0)_c = sum over L of wc (1 - r); the
  // exponentials of all rows first (independent chains), then sums and stores
  const double *rr = a.r + tok_base(a.t, b, g);
  double om[TPL];                           // 1 - r on L, 0 on the resident set and past n
#pragma unroll
  for (int u = 0; u < TPL; ++u) {
    const int tok = base + lane + u * WAVE;
    const double rv = tok < n ? rr[tok] : 1.0;
    om[u] = rv < 1.0 ? 1.0 - rv : 0.0;
  }
  double ev[G][TPL];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int u = 0; u < TPL; ++u) ev[j][u] = exp(sc[j][lane + u * WAVE] - mrow[j]);
  double part[2 * G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    double sum = 0.0, f0 = 0.0;
#pragma unroll
    for (int u = 0; u < TPL; ++u) { sum += ev[j][u]; f0 += ev[j][u] * om[u]; }
    part[2 * j] = sum;
    part[2 * j + 1] = f0;
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    double *wrow = a.wc + row_tok_base(a.t, b, g * G + j) + base;
#pragma unroll
    for (int u = 0; u < TPL; ++u)
      if (base + lane + u * WAVE < n) wrow[lane + u * WAVE] = ev[j][u];
  }
#pragma unroll
  for (int k = 0; k < 2 * G; ++k) part[k] = wave_sum(part[k]);
  if (lane < G) {
    double pm = mrow[0], ps = part[0], pf = part[1];
#pragma unroll
    for (int j = 1; j < G; ++j)
      if (lane == j) { pm = mrow[j]; ps = part[2 * j]; pf = part[2 * j + 1]; }
    const int64_t o = row_chunk_base(a.t, b, g * G + lane) + c;
    a.cstat[o] = make_double2(pm, ps);
    a.cf0[o] = pf;
  }
}

template <bool BF16, int G>
static hipError_t launch_sketch_t(const SketchArgs &a, hipStream_t st) {
  const int blocks = (a.total_blocks + SK_WAVES - 1) / SK_WAVES;
  if (a.q2) return launch_kernel(k_sketch<false, G, true>, dim3(blocks), dim3(SK_WAVES * WAVE), 0, st, a);
  return launch_kernel(k_sketch<BF16, G>, dim3(blocks), dim3(SK_WAVES * WAVE), 0, st, a);
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
