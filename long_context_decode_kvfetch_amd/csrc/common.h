// Internal device/host helpers shared by the VerKV kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/verkv.h"

namespace verkv {

constexpr int D = VERKV_HEAD_DIM;          // head dimension
constexpr int SKETCH_CHUNK = 128;          // tokens per sketch-scoring wave
constexpr int WAVE = 64;

// Per-sequence offsets of a ragged batch, passed by value in kernel arguments.  A
// sequence's token arrays are strided by its capacity (>= its length), so a sequence
// can grow in place; with no capacity given the capacity is the length.
struct SeqInfo {
  int32_t n;          // tokens
  int32_t cap;        // token capacity: the stride of the sequence's per-head arrays
  int32_t tok_off;    // sum of cap over earlier sequences
  int32_t word_off;   // sum of ceil(cap/32) over earlier sequences
  int32_t chunk_off;  // sum of ceil(cap/SKETCH_CHUNK) over earlier sequences
};
struct SeqTable {
  int32_t B;
  int32_t Hkv;
  int32_t G;
  int32_t n_sink;
  int32_t n_local;
  int32_t max_n;
  int32_t max_cap;
  SeqInfo s[VERKV_MAX_BATCH];
  uint8_t order[VERKV_MAX_BATCH];   // sequences by length, longest first (ties by index):
                                    // the order row-per-workgroup launches dispatch them
  int32_t tok_bits;                 // bits of a token id in a host-row list entry (the
                                    // largest capacity's), the prefetch slot + 1 above them
  int32_t stage_slots;              // staging slots per KV head asked for (0: default)
};

// A host-row list entry: token | (prefetch slot + 1) << tok_bits, as uint32.
__host__ __device__ inline int entry_token(int32_t e, int tb) {
  return (int)((uint32_t)e & ((1u << tb) - 1u));
}
__host__ __device__ inline int entry_slot(int32_t e, int tb) {   // -1: not prefetched
  return (int)((uint32_t)e >> tb) - 1;
}

__host__ __device__ inline int32_t words_of(int32_t n) { return (n + 31) >> 5; }
__host__ __device__ inline int32_t chunks_of(int32_t n) { return (n + SKETCH_CHUNK - 1) / SKETCH_CHUNK; }

// Offsets of unit (b, g) and of query row (b, h) in the layouts of verkv.h.
__host__ __device__ inline int64_t tok_base(const SeqTable &t, int b, int g) {
  return (int64_t)t.Hkv * t.s[b].tok_off + (int64_t)g * t.s[b].cap;
}
__host__ __device__ inline int64_t word_base(const SeqTable &t, int b, int g) {
  return (int64_t)t.Hkv * t.s[b].word_off + (int64_t)g * words_of(t.s[b].cap);
}
__host__ __device__ inline int64_t row_tok_base(const SeqTable &t, int b, int h) {
  return (int64_t)t.Hkv * t.G * t.s[b].tok_off + (int64_t)h * t.s[b].cap;
}
__host__ __device__ inline int64_t row_chunk_base(const SeqTable &t, int b, int h) {
  return (int64_t)t.Hkv * t.G * t.s[b].chunk_off + (int64_t)h * chunks_of(t.s[b].cap);
}

// ------------------------------------------------------------------ cross-lane helpers
// DPP patterns within a row of 16 lanes (gfx9 encodings).
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7-i within each half row
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15-i within the row
constexpr int DPP_ROR8 = 0x128;        // row_ror:8 -> lane i <-> i ^ 8 within a 16-lane row
constexpr int DPP_ROW_BCAST0 = 0x150;  // row_newbcast:n (+ n): lane n of each row to the whole row

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
  int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}

// Butterfly sums over each row of 16 lanes; every lane of the row gets the same value
// (each step adds a commuted pair, so the association is identical in all lanes).
__device__ __forceinline__ double sum16(double v) {
  v += dpp_d<DPP_XOR1>(v);
  v += dpp_d<DPP_XOR2>(v);
  v += dpp_d<DPP_HALF_MIRROR>(v);
  v += dpp_d<DPP_MIRROR>(v);
  return v;
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f<DPP_XOR1>(v);
  v += dpp_f<DPP_XOR2>(v);
  v += dpp_f<DPP_HALF_MIRROR>(v);
  v += dpp_f<DPP_MIRROR>(v);
  return v;
}

__device__ __forceinline__ double shfl_xor_d(double v, int m) { return __shfl_xor(v, m, WAVE); }
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, WAVE); }

__device__ __forceinline__ double wave_sum(double v) {
  v = sum16(v);
  v += shfl_xor_d(v, 16);
  v += shfl_xor_d(v, 32);
  return v;
}

__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
  for (int m = 1; m < WAVE; m <<= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  for (int m = 1; m < WAVE; m <<= 1) {
    uint64_t o = __shfl_xor(v, m, WAVE);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ double max16(double v) {
  v = fmax(v, dpp_d<DPP_XOR1>(v));
  v = fmax(v, dpp_d<DPP_XOR2>(v));
  v = fmax(v, dpp_d<DPP_HALF_MIRROR>(v));
  v = fmax(v, dpp_d<DPP_MIRROR>(v));
  return v;
}
__device__ __forceinline__ double min16(double v) {
  v = fmin(v, dpp_d<DPP_XOR1>(v));
  v = fmin(v, dpp_d<DPP_XOR2>(v));
  v = fmin(v, dpp_d<DPP_HALF_MIRROR>(v));
  v = fmin(v, dpp_d<DPP_MIRROR>(v));
  return v;
}

// wave-wide maximum / minimum: DPP inside each row of 16 lanes, then two shuffles
__device__ __forceinline__ double wave_max(double v) {
  v = max16(v);
  v = fmax(v, shfl_xor_d(v, 16));
  return fmax(v, shfl_xor_d(v, 32));
}
__device__ __forceinline__ double wave_min(double v) {
  v = min16(v);
  v = fmin(v, shfl_xor_d(v, 16));
  return fmin(v, shfl_xor_d(v, 32));
}

// Block-wide reductions in a fixed order (deterministic): each wave reduces, lane k of
// every wave then reads wave k's partial and a 16-lane butterfly finishes, so every
// thread holds the same result and only one partial per quantity is live per lane.
// `scratch` holds one entry per wave (at most 16 waves).  Ends with a barrier so the
// scratch may be reused immediately.
template <int NT>
__device__ __forceinline__ double block_sum(double v, double *scratch) {
  constexpr int NW = NT / WAVE;
  static_assert(NW <= 16, "at most 16 waves");
  v = wave_sum(v);
  const int lane = threadIdx.x & (WAVE - 1);
  if (lane == 0) scratch[threadIdx.x / WAVE] = v;
  __syncthreads();
  const int k = lane & 15;
  double t = k < NW ? scratch[k] : 0.0;
  t = sum16(t);
  __syncthreads();
  return t;
}
template <int NT>
__device__ __forceinline__ double block_max(double v, double *scratch) {
  constexpr int NW = NT / WAVE;
  static_assert(NW <= 16, "at most 16 waves");
  v = wave_max(v);
  const int lane = threadIdx.x & (WAVE - 1);
  if (lane == 0) scratch[threadIdx.x / WAVE] = v;
  __syncthreads();
  const int k = lane & 15;
  double t = k < NW ? scratch[k] : -INFINITY;
  t = max16(t);
  __syncthreads();
  return t;
}
template <int NT>
__device__ __forceinline__ double block_min(double v, double *scratch) {
  constexpr int NW = NT / WAVE;
  static_assert(NW <= 16, "at most 16 waves");
  v = wave_min(v);
  const int lane = threadIdx.x & (WAVE - 1);
  if (lane == 0) scratch[threadIdx.x / WAVE] = v;
  __syncthreads();
  const int k = lane & 15;
  double t = k < NW ? scratch[k] : INFINITY;
  t = min16(t);
  __syncthreads();
  return t;
}
template <int NT>
__device__ __forceinline__ int64_t block_sum_i64(int64_t v, int64_t *scratch) {
  constexpr int NW = NT / WAVE;
  v = wave_sum_i64(v);
  const int w = threadIdx.x / WAVE;
  if ((threadIdx.x & (WAVE - 1)) == 0) scratch[w] = v;
  __syncthreads();
  int64_t t = 0;
#pragma unroll 1
  for (int i = 0; i < NW; ++i) t += scratch[i];
  __syncthreads();
  return t;
}

// Exclusive prefix sum of one int per thread over the block, in thread order.
template <int NT>
__device__ __forceinline__ int32_t block_excl_scan(int32_t v, int32_t *scratch, int32_t *total) {
  constexpr int NW = NT / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  const int w = threadIdx.x / WAVE;
  int32_t incl = v;
  for (int off = 1; off < WAVE; off <<= 1) {
    int32_t o = __shfl_up(incl, off, WAVE);
    if (lane >= off) incl += o;
  }
  if (lane == WAVE - 1) scratch[w] = incl;
  __syncthreads();
  int32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if (i < w) before += scratch[i];
    all += scratch[i];
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// bf16 pairs packed in a 32-bit word: element 2k in the low half, 2k+1 in the high half.
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// A 16-byte load with the streaming (non-temporal) cache policy, for data read once
// per step: the lines are not kept in the caches for reuse.
__device__ __forceinline__ uint4 load_stream16(const uint8_t *p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Load the 16-byte slice of a cache row that a lane owns and widen it to float.
// bf16 rows: 8 elements per lane; f32 rows: 4 elements per lane.
template <bool BF16>
struct RowSlice;
template <>
struct RowSlice<true> {
  static constexpr int EPL = 8;
  __device__ __forceinline__ static void widen(const uint4 &u, float *x) {
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x);
    x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
    x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z);
    x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
  }
};
template <>
struct RowSlice<false> {
  static constexpr int EPL = 4;
  __device__ __forceinline__ static void widen(const uint4 &u, float *x) {
    x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
  }
};

// ------------------------------------------------------------------ Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).
struct Philox4 { uint32_t x0, x1, x2, x3; };
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd) { k0 += W0; k1 += W1; }
    const uint32_t lo0 = M0 * c0, hi0 = __umulhi(M0, c0);
    const uint32_t lo1 = M1 * c2, hi1 = __umulhi(M1, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return {c0, c1, c2, c3};
}
// 53-bit uniform in [0,1): ((x0 * 2^32 + x1) >> 11) * 2^-53.
__device__ __forceinline__ double philox_uniform53(uint32_t tok, uint32_t head, uint32_t layer,
                                                   uint32_t stream, uint64_t seed) {
  const Philox4 p = philox4x32_10(tok, head, layer, stream, (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint64_t top = ((((uint64_t)p.x0) << 32) | p.x1) >> 11;
  return (double)top * 0x1.0p-53;
}

}  // namespace verkv
