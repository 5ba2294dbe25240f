// The 2-bit key sketch for gfx950: asymmetric uniform quantisation of every key row in
// groups of 32 dimensions (the pages evaluate KVFetch with a 2-bit sketch, "Verify
// Before You Fetch", picx.dev summary page, evaluation of the error-bound guarantee, but
// define no quantiser; the per-token grouping is the one of KIVI, on the pages' list of
// related work).  Per group: mn = min, sc = (max - min) / 3 in float32, code = the
// number of midpoints mn + (c + 1/2) sc (c = 0, 1, 2, float64) the value reaches.
//
// One token row per 16 lanes, each lane an 8-dimension piece; the four lanes of a group
// form a DPP quad, so the group's min and max are two quad exchanges.  Output row (64
// bytes): eight words, word w = codes of piece w | codes of piece w + 8 << 16, then
// (mn, sc) of groups 0, 2, 1, 3 as float32 (the order the sketch kernel's lanes read).
#include "kernels.h"

namespace verkv {

constexpr int QT_NT = 256;
constexpr int QT_ROWS = QT_NT / 16;       // token rows per workgroup

template <bool BF16>
__global__ __launch_bounds__(QT_NT) void k_quant_sketch(QuantArgs a) {
  constexpr int ROW_BYTES = D * (BF16 ? 2 : 4);
  const int sub = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * QT_ROWS + threadIdx.x / 16;
  const bool valid = row < a.rows;
  const int64_t rr = valid ? row : a.rows - 1;     // every lane takes part in the exchanges
  float x[8];
  const uint8_t *src = a.K + rr * ROW_BYTES + (int64_t)sub * 8 * (BF16 ? 2 : 4);
  if constexpr (BF16) {
    RowSlice<true>::widen(*(const uint4 *)src, x);
  } else {
    RowSlice<false>::widen(*(const uint4 *)src, x);
    RowSlice<false>::widen(*(const uint4 *)(src + 16), x + 4);
  }
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) {
    mn = fminf(mn, x[e]);
    mx = fmaxf(mx, x[e]);
  }
  mn = fminf(mn, dpp_f<DPP_XOR1>(mn));
  mx = fmaxf(mx, dpp_f<DPP_XOR1>(mx));
  mn = fminf(mn, dpp_f<DPP_XOR2>(mn));
  mx = fmaxf(mx, dpp_f<DPP_XOR2>(mx));
  const float sc = (mx - mn) / 3.0f;               // IEEE float32 subtraction and division
  const double m64 = (double)mn, s64 = (double)sc;
  const double t0 = m64 + 0.5 * s64, t1 = m64 + 1.5 * s64, t2 = m64 + 2.5 * s64;
  uint32_t code = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double v = (double)x[e];
    const uint32_t c = (v >= t0 ? 1u : 0u) + (v >= t1 ? 1u : 0u) + (v >= t2 ? 1u : 0u);
    code |= c << (2 * e);
  }
  const uint32_t hi = (uint32_t)__shfl_xor((int)code, 8, 16);     // piece sub ^ 8
  if (!valid) return;
  uint8_t *dst = a.out + row * SKETCH2_ROW_BYTES;
  if (sub < 8) *(uint32_t *)(dst + 4 * sub) = code | (hi << 16);
  if ((sub & 3) == 0) {
    const int g = sub >> 2;
    const int fi = (g & 1) * 4 + (g >> 1) * 2;
    *(float2 *)(dst + 32 + 4 * fi) = make_float2(mn, sc);
  }
}

hipError_t launch_quant_sketch(const QuantArgs &a, bool bf16, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  const int64_t blocks = (a.rows + QT_ROWS - 1) / QT_ROWS;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (bf16) return launch_kernel(k_quant_sketch<true>, dim3((unsigned)blocks), dim3(QT_NT), 0, st, a);
  return launch_kernel(k_quant_sketch<false>, dim3((unsigned)blocks), dim3(QT_NT), 0, st, a);
}

}  // namespace verkv
