// Kernel arguments of the forward pass (host and device).
#pragma once

#include "common.hpp"

namespace attn119 {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N;
  int Hkv;            // key/value heads (H_kv divides H; query head h reads h / (H / Hkv))
  int nqb;            // ceil(N / 128) query blocks = key blocks
  float c;            // scale * log2(e)
  float sc2;          // softcap: 2 * scale * log2(e) / cap
  float cap2;         // softcap: cap * log2(e)
  float tau;          // rescale threshold (log2 units)
  float alibi_exp;    // default slopes: slope_h = exp2(alibi_exp * (h + 1)), alibi_exp = -8/H
  const float* alibi_slopes;  // [H] or null
  const float* q_scale;       // fp8: [B][H][nqb]
  const float* k_scale;
  const float* v_scale;
  const unsigned char* map;   // block map (masked variants)
  MapLayout lay;
  int compact;                // 1: the map is the compact form (a packed batch's workspace)
  uint32_t mflags;            // positional mask flags the map was built for
  int window;
  int order;                  // work order: kOrderHeadMajor or kOrderHeavyFirst
  int* rescale_counts;        // [B][H][N] rescale events per query row, or null (not counted)
};

// Order in which workgroups take (b*H + h, row block) work items.  Workgroup L runs on
// XCD L % 8 (the dispatcher deals workgroups round-robin over the 8 XCDs).
//  kOrderHeadMajor : each XCD takes a contiguous range of items, head by head, a head's
//                    row blocks last-first -- the row blocks sharing a head's K/V run
//                    on one XCD at the same time (L2 reuse).
//  kOrderHeavyFirst: items in row-block-major order, last row block first: under a
//                    causal mask the last row blocks carry the most key blocks, so this
//                    is longest-first list scheduling, which evens out the finish times
//                    when there are only a few workgroups per slot.  With B*H a multiple
//                    of 8 a head still stays on one XCD, and so does a run of
//                    consecutive heads.
//  kOrderMapSorted : document masks, where a row block's work depends on where it sits
//                    in its document: the block map's work-order section lists the
//                    (batch row, row block) pairs heaviest-first, and workgroup L takes
//                    pair order[L / H] of head L % H (H a multiple of 8: XCD x takes the
//                    contiguous heads x*H/8 .. (x+1)*H/8-1 of every batch row).
constexpr int kOrderHeadMajor = 0, kOrderHeavyFirst = 1, kOrderMapSorted = 2;

// Flat key/value head index (b * Hkv + key/value head) of flat query head bh = b * H + h.
__device__ __forceinline__ int kv_head(const FwdArgs& a, int bh) {
  const int b = bh / a.H, h = bh - b * a.H;
  return b * a.Hkv + h / (a.H / a.Hkv);
}

__device__ __forceinline__ void work_item(const FwdArgs& a, int L, int& bh, int& qb) {
  const int nqb = a.nqb;
  if (a.order == kOrderMapSorted) {
    const int H = a.H, M = a.B * nqb;
    const int r = L / H;
    const int i = L - r * H;
    const int h = (H & 7) ? i : (i & 7) * (H >> 3) + (i >> 3);
    // a map that fails its header check (it is then ignored and the outputs poisoned)
    // falls back to the identity order, so every work item is still visited once
    typedef const __attribute__((address_space(4))) int cint;
    const __attribute__((address_space(4))) MapHeader* hd =
        (const __attribute__((address_space(4))) MapHeader*)a.map;
    const bool ok = hd->magic == kMapMagic && hd->B == a.B && hd->N == a.N;
    const int e = ok ? min(max(((cint*)(a.map + a.lay.order))[r], 0), M - 1) : r;
    const int b = e / nqb;
    bh = b * H + h;
    qb = e - b * nqb;
  } else if (a.order == kOrderHeavyFirst) {
    const int BH = a.B * a.H;
    const int r = L / BH;
    const int i = L - r * BH;
    // With B*H a multiple of 8, XCD x takes the contiguous heads x*BH/8 .. (x+1)*BH/8-1,
    // so the query heads of one key/value group share that XCD's L2.
    bh = (BH & 7) ? i : (i & 7) * (BH >> 3) + (i >> 3);
    qb = nqb - 1 - r;
  } else {
    const int T = a.B * a.H * nqb;
    const int xcd = L & 7, jx = L >> 3;
    const int wid = xcd * (T >> 3) + min(xcd, T & 7) + jx;
    bh = wid / nqb;
    qb = nqb - 1 - (wid - bh * nqb);
  }
}

}  // namespace attn119
