// Host-row prefetch for gfx950: between two decode steps of a layer the fetch sets
// overlap heavily, so the rows the previous step read from the host (KVFetch
// step 5, "Verify Before You Fetch", picx.dev summary page) are copied into the
// workspace while the current step's decision kernel runs; the host-row kernel of the
// current step takes those it needs from there instead of the host link.  The values
// are the same rows of the same cache, so results do not change.
#include "kernels.h"

#include <algorithm>

namespace verkv {

// ------------------------------------------------------------------ host-row prefetch
// Stages, per KV head, the value rows of the first stage_rows entries of the previous
// step's host-row list in the workspace (three rows in flight per lane group), records
// each slot's token, and sets the token's bit in the head's bitmask of prefetched
// tokens (cleared by the sketch kernel of the same step; an OR per staged row, so the
// mask does not depend on the order the rows are staged in).  Two staging buffers alternate: a row the previous step staged is copied
// from the other buffer (device memory; the list entry carries its slot there), only the
// others are read from the pinned host cache (zero-copy loads), so the host link carries
// the rows that are new to the list.
// The other buffer is trusted only when the staging header names this cache (its
// device address and a hash of the shape, published by the list kernel of the previous
// step); otherwise every row comes from the host.  Entries are validated (token < n),
// so a list left by another shape only costs useless copies.  The kernel runs beside
// the decision kernel (one 256-thread block per CU fits next to it: no LDS, at most 32
// VGPRs), so it lives in a file of its own.
constexpr int PF_NT = 256;
constexpr int PF_GRID = 256;               // blocks per launch: at most one per CU, so each
                                           // fits beside a decision-kernel workgroup

// With a key cache (krows: the sketch is not exact, so the host-row kernel scores the
// fetched rows from the host keys) a slot holds the value row and then the key row,
// and both come from the other buffer or the host together.
template <bool BF16, bool KV>
__global__ __launch_bounds__(PF_NT) __attribute__((amdgpu_num_vgpr(32))) void k_prefetch(PrefetchArgs a) {
  using RS = RowSlice<BF16>;
  constexpr int LPR = D / RS::EPL;         // lanes per row (16 or 32)
  constexpr int RPI = PF_NT / LPR;         // rows per block iteration
  constexpr int ROW_BYTES = D * (BF16 ? 2 : 4);
  constexpr int INFL = KV ? 1 : 2;         // slots in flight per lane group
  const int unit = blockIdx.y;
  const int b = unit / a.t.Hkv;
  const int g = unit % a.t.Hkv;
  const int n = a.t.s[b].n;
  const int tid = threadIdx.x;
  const int cnt = min(max(a.prev_count[unit], 0), n);
  const int ns = min(cnt, a.stage_rows);
  const int32_t *pl = a.prev_list + tok_base(a.t, b, g);
  uint32_t *sb = a.sbits + word_base(a.t, b, g);
  const int sub = tid % LPR;
  const int64_t src = tok_base(a.t, b, g);
  const int64_t SS = a.stage_stride;
  // which buffer to write, and whether the other one holds rows of this cache
  const uint64_t *h = a.shdr;
  const bool have_old = h && h[0] == STAGE_MAGIC && h[1] == a.ident_ptr &&
                        h[2] == a.ident_shape && h[3] <= 1;
  const int cur = have_old ? 1 - (int)h[3] : 0;
  if (h && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) a.shdr[4] = (uint64_t)cur;
  const int64_t ubase = (int64_t)unit * a.stage_rows;
  uint8_t *dst = (cur ? a.stage_alt : a.stage) + ubase * SS;
  int32_t *dtok = (cur ? a.stage_tok_alt : a.stage_tok) + ubase;
  const uint8_t *osrc = (cur ? a.stage : a.stage_alt) + ubase * SS;
  const uint32_t *otok = reinterpret_cast<const uint32_t *>((cur ? a.stage_tok : a.stage_tok_alt) + ubase);
  // slots in flight per lane group in named registers (an indexed array here would be
  // placed in LDS, which must stay free for the decision kernel beside this one)
  // an entry of the previous list carries the slot its token had in the buffer the
  // previous step staged (the other buffer now), checked against that slot's token
  auto fetch = [&](int p, uint4 &v, uint4 &k) -> int {
    if (p >= ns) return -1;
    const int32_t e = pl[p];
    const int tok = entry_token(e, a.t.tok_bits);
    if (tok >= n) return -1;
    const int j = entry_slot(e, a.t.tok_bits);
    if (have_old && j >= 0 && j < a.stage_rows && otok[j] == (uint32_t)tok) {
      const uint8_t *o = osrc + (int64_t)j * SS + sub * 16;
      v = *(const uint4 *)o;
      if (KV) k = *(const uint4 *)(o + ROW_BYTES);
    } else {
      v = *(const uint4 *)(a.vrows + (src + tok) * ROW_BYTES + sub * 16);
      if (KV) k = *(const uint4 *)(a.krows + (src + tok) * ROW_BYTES + sub * 16);
    }
    return tok;
  };
  auto put = [&](int p, int tok, const uint4 &v, const uint4 &k) {
    if (p >= a.stage_rows) return;
    if (tok >= 0) {
      uint8_t *d = dst + (int64_t)p * SS + sub * 16;
      *(uint4 *)d = v;
      if (KV) *(uint4 *)(d + ROW_BYTES) = k;
    }
    if (sub == 0) {
      dtok[p] = tok;
      if (tok >= 0) atomicOr(sb + (tok >> 5), 1u << (tok & 31));
    }
  };
  for (int p0 = blockIdx.x * RPI * INFL; p0 < a.stage_rows; p0 += gridDim.x * RPI * INFL) {
    const int pa = p0 + tid / LPR;
    uint4 va = make_uint4(0, 0, 0, 0), ka = va;
    const int ta = fetch(pa, va, ka);
    if constexpr (KV) {
      put(pa, ta, va, ka);
    } else {
      const int pb = pa + RPI;
      uint4 vb = make_uint4(0, 0, 0, 0);
      const int tb = fetch(pb, vb, ka);
      put(pa, ta, va, ka);
      put(pb, tb, vb, ka);
    }
  }
}

hipError_t launch_prefetch(const PrefetchArgs &a, int units, bool bf16, hipStream_t st) {
  const int per_unit = std::max(1, PF_GRID / std::max(1, units));
  const dim3 grid(per_unit, units);
  if (a.krows) {
    if (bf16) return launch_kernel(k_prefetch<true, true>, grid, dim3(PF_NT), 0, st, a);
    return launch_kernel(k_prefetch<false, true>, grid, dim3(PF_NT), 0, st, a);
  }
  if (bf16) return launch_kernel(k_prefetch<true, false>, grid, dim3(PF_NT), 0, st, a);
  return launch_kernel(k_prefetch<false, false>, grid, dim3(PF_NT), 0, st, a);
}

}  // namespace verkv
