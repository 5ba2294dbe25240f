// Host-row staging for gfx950: between two decode steps of a layer the fetch sets
// overlap heavily, so the rows the previous step read from the host (KVFetch step 5,
// "Verify Before You Fetch", picx.dev summary page) are kept in the workspace, and the
// host-row kernel of the current step takes those it needs from there instead of the
// host link.  The values are the same rows of the same cache, so results do not change.
//
// The staging area of a KV head is a set of slots that keep their rows from step to
// step.  Each step makes the tokens of the first stage_rows entries of the previous
// step's host-row list resident: a token already in a slot stays there and costs
// nothing; the others are read from the pinned host cache (zero-copy loads) into slots
// whose tokens that list no longer holds, in slot order.  Two maps, slot -> token
// (stage_tok) and token -> slot (slot_of), describe the area; a pair that does not agree
// is not a staged row, so a map left by anything else only costs host reads.
//
// Two kernels on the library's second stream.  The plan (one workgroup per KV head:
// which tokens come in, which slots they take, which tokens leave) needs no host link,
// so it runs at the end of a step, beside that step's host-row kernel, as soon as the
// list exists.  The row copies need the link, so they run in the next step beside its
// decision kernel, when the link is idle.  The staging header records for which cache
// the maps hold rows (published by the list kernel after a step whose copies ran) and
// for which cache the pending plan was made (written by the plan): the copies run only
// for the cache the plan was made for, and the plan clears the maps first when they
// belong to another cache.  The plan may empty slots (their token leaving) while the
// host-row kernel of its step reads the area; such a row is then read from the host,
// where it has the same value.
#include "kernels.h"

#include <algorithm>

namespace verkv {

constexpr int SP_NT = 1024;                // plan: one workgroup per KV head
constexpr int SP_B = 8;                    // plan: entries or slots per batch of loads
constexpr int PF_NT = 256;
constexpr int PF_GRID = 48;                // copy blocks per launch: enough rows in flight for
                                           // the link, few CUs taken from the decision kernel

__global__ __launch_bounds__(SP_NT) void k_stage_plan(PrefetchArgs a) {
  extern __shared__ uint32_t s_keep[];     // [ceil(S / 32)] slots the list keeps
  __shared__ int32_t iscr[SP_NT / WAVE];
  const int unit = blockIdx.x;
  const int b = unit / a.t.Hkv;
  const int g = unit % a.t.Hkv;
  const int n = a.t.s[b].n;
  const int cap = a.t.s[b].cap;
  const int S = a.stage_rows;
  const int KW = (S + 31) / 32;
  const int tid = threadIdx.x;
  int32_t *stok = a.stage_tok + (int64_t)unit * S;
  int32_t *smap = a.slot_of + tok_base(a.t, b, g);
  int32_t *pnew = a.pf_new + (int64_t)unit * S;
  int32_t *pslot = a.pf_slot + (int64_t)unit * S;
  uint64_t *h = a.shdr;
  const bool have = h[0] == STAGE_MAGIC && h[1] == a.ident_ptr && h[2] == a.ident_shape;
  if (!have) {                             // maps of another cache, or none: clear them
    for (int s = tid; s < S; s += SP_NT) stok[s] = -1;
    for (int i = tid; i < cap; i += SP_NT) smap[i] = -1;
  }
  for (int w = tid; w < KW; w += SP_NT) s_keep[w] = 0u;
  __syncthreads();

  // The list's first entries, a contiguous run per thread, in batches whose loads are
  // all issued before any is used: a token some slot holds (both maps agree) keeps its
  // slot; the others are new.  pslot[p] holds the new token or -1 until the slots are
  // assigned below.
  const int cnt = min(max(a.prev_count[unit], 0), n);
  const int ns = min(cnt, S);
  const int32_t *pl = a.prev_list + tok_base(a.t, b, g);
  const int per = (ns + SP_NT - 1) / SP_NT;
  const int e0 = min(ns, tid * per), e1 = min(ns, e0 + per);
  int mine = 0;
  for (int p0 = e0; p0 < e1; p0 += SP_B) {
    int tok[SP_B], j[SP_B], held[SP_B];
#pragma unroll
    for (int u = 0; u < SP_B; ++u) {
      tok[u] = p0 + u < e1 ? entry_token(pl[p0 + u], a.t.tok_bits) : n;
      if (tok[u] >= n) tok[u] = -1;        // past the run, or not a token of this sequence
    }
#pragma unroll
    for (int u = 0; u < SP_B; ++u) j[u] = tok[u] >= 0 ? smap[tok[u]] : -1;
#pragma unroll
    for (int u = 0; u < SP_B; ++u) held[u] = (j[u] >= 0 && j[u] < S) ? stok[j[u]] : -2;
#pragma unroll
    for (int u = 0; u < SP_B; ++u) {
      if (p0 + u >= e1) break;
      const bool keep = tok[u] >= 0 && held[u] == tok[u];
      if (keep) atomicOr(&s_keep[j[u] >> 5], 1u << (j[u] & 31));
      const bool fresh = tok[u] >= 0 && !keep;
      pslot[p0 + u] = fresh ? tok[u] : -1;
      mine += fresh ? 1 : 0;
    }
  }
  int32_t nnew = 0;
  int32_t k = block_excl_scan<SP_NT>(mine, iscr, &nnew);   // its barriers publish s_keep
  for (int p0 = e0; p0 < e1; p0 += SP_B) {
    int nt[SP_B];
#pragma unroll
    for (int u = 0; u < SP_B; ++u) nt[u] = p0 + u < e1 ? pslot[p0 + u] : -1;   // own writes
#pragma unroll
    for (int u = 0; u < SP_B; ++u)
      if (nt[u] >= 0) pnew[k++] = nt[u];
  }
  // free slots in slot order, a contiguous run per thread: the first nnew of them take
  // the new tokens, and the tokens they held leave
  const int sp = (S + SP_NT - 1) / SP_NT;
  const int s0 = min(S, tid * sp), s1 = min(S, s0 + sp);
  auto kept = [&](int s) { return (s_keep[s >> 5] >> (s & 31)) & 1u; };
  int nfree = 0;
  for (int s = s0; s < s1; ++s) nfree += kept(s) ? 0 : 1;
  int32_t tfree = 0;
  // its barriers also keep every read of pslot above before the writes below
  int32_t f = block_excl_scan<SP_NT>(nfree, iscr, &tfree);
  for (int q0 = s0; q0 < s1 && f < nnew; q0 += SP_B) {
    int old[SP_B], back[SP_B];
#pragma unroll
    for (int u = 0; u < SP_B; ++u) old[u] = (q0 + u < s1 && !kept(q0 + u)) ? stok[q0 + u] : -1;
#pragma unroll
    for (int u = 0; u < SP_B; ++u) back[u] = (old[u] >= 0 && old[u] < cap) ? smap[old[u]] : -1;
#pragma unroll
    for (int u = 0; u < SP_B; ++u) {
      const int s = q0 + u;
      if (s >= s1 || f >= nnew) break;
      if (kept(s)) continue;
      if (old[u] >= 0 && old[u] < cap && back[u] == s) smap[old[u]] = -1;
      stok[s] = -1;
      pslot[f++] = s;
    }
  }
  if (tid == 0) a.pf_count[unit] = min(nnew, tfree);
  if (blockIdx.x == 0 && tid == 0) {       // the plan is for this cache
    h[3] = a.ident_ptr;
    h[4] = a.ident_shape;
    h[5] = PLAN_MAGIC;
  }
}

// The rows the pending plan brings in, when it was made for this cache: per lane group
// one slot (two in flight without keys), value row then key row; the slot's maps are
// written after its row.  Header word 6 tells the list kernel whether the copies ran.
template <bool BF16, bool KV>
__global__ __launch_bounds__(PF_NT) __attribute__((amdgpu_num_vgpr(32))) void k_stage_fetch(PrefetchArgs a) {
  using RS = RowSlice<BF16>;
  constexpr int LPR = D / RS::EPL;         // lanes per row (16 or 32)
  constexpr int RPI = PF_NT / LPR;         // rows per block iteration
  constexpr int ROW_BYTES = D * (BF16 ? 2 : 4);
  constexpr int INFL = KV ? 1 : 2;         // slots in flight per lane group
  const uint64_t *h = a.shdr;
  const bool planned = h[5] == PLAN_MAGIC && h[3] == a.ident_ptr && h[4] == a.ident_shape;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.shdr[6] = planned ? 1ull : 0ull;
  if (!planned) return;
  const int unit = blockIdx.y;
  const int b = unit / a.t.Hkv;
  const int g = unit % a.t.Hkv;
  const int n = a.t.s[b].n;
  const int S = a.stage_rows;
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  const int cnt = min(a.pf_count[unit], S);
  const int32_t *pnew = a.pf_new + (int64_t)unit * S;
  const int32_t *pslot = a.pf_slot + (int64_t)unit * S;
  int32_t *stok = a.stage_tok + (int64_t)unit * S;
  int32_t *smap = a.slot_of + tok_base(a.t, b, g);
  const int64_t src = tok_base(a.t, b, g);
  const int64_t SS = a.stage_stride;
  uint8_t *area = a.stage + (int64_t)unit * S * SS;
  // slots in flight per lane group in named registers (an indexed array here would be
  // placed in LDS, which must stay free for the decision kernel beside this one)
  auto fetch = [&](int k, uint4 &v, uint4 &kr) -> int {
    if (k >= cnt) return -1;
    const int tok = pnew[k];
    if (tok < 0 || tok >= n) return -1;
    v = *(const uint4 *)(a.vrows + (src + tok) * ROW_BYTES + sub * 16);
    if (KV) kr = *(const uint4 *)(a.krows + (src + tok) * ROW_BYTES + sub * 16);
    return tok;
  };
  auto put = [&](int k, int tok, const uint4 &v, const uint4 &kr) {
    if (tok < 0) return;
    const int s = pslot[k];
    if (s < 0 || s >= S) return;
    uint8_t *d = area + (int64_t)s * SS + sub * 16;
    *(uint4 *)d = v;
    if (KV) *(uint4 *)(d + ROW_BYTES) = kr;
    if (sub == 0) {
      stok[s] = tok;
      smap[tok] = s;
    }
  };
  for (int k0 = blockIdx.x * RPI * INFL; k0 < cnt; k0 += gridDim.x * RPI * INFL) {
    const int ka = k0 + tid / LPR;
    uint4 va = make_uint4(0, 0, 0, 0), kra = va;
    const int ta = fetch(ka, va, kra);
    if constexpr (KV) {
      put(ka, ta, va, kra);
    } else {
      const int kb = ka + RPI;
      uint4 vb = make_uint4(0, 0, 0, 0);
      const int tb = fetch(kb, vb, kra);
      put(ka, ta, va, kra);
      put(kb, tb, vb, kra);
    }
  }
}

hipError_t launch_stage_plan(const PrefetchArgs &a, int units, hipStream_t st) {
  const size_t keep = 4 * (size_t)((a.stage_rows + 31) / 32);
  return launch_kernel(k_stage_plan, dim3(units), dim3(SP_NT), (uint32_t)keep, st, a);
}

hipError_t launch_stage_fetch(const PrefetchArgs &a, int units, bool bf16, hipStream_t st) {
  const int per_unit = std::max(1, PF_GRID / std::max(1, units));
  const dim3 grid(per_unit, units);
  if (a.krows) {
    if (bf16) return launch_kernel(k_stage_fetch<true, true>, grid, dim3(PF_NT), 0, st, a);
    return launch_kernel(k_stage_fetch<false, true>, grid, dim3(PF_NT), 0, st, a);
  }
  if (bf16) return launch_kernel(k_stage_fetch<true, false>, grid, dim3(PF_NT), 0, st, a);
  return launch_kernel(k_stage_fetch<false, false>, grid, dim3(PF_NT), 0, st, a);
}

}  // namespace verkv
