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
  uint32_t mflags;            // positional mask flags the map was built for
  int window;
  int order;                  // work order: kOrderHeadMajor or kOrderHeavyFirst
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
constexpr int kOrderHeadMajor = 0, kOrderHeavyFirst = 1;

// Flat key/value head index (b * Hkv + key/value head) of flat query head bh = b * H + h.
__device__ __forceinline__ int kv_head(const FwdArgs& a, int bh) {
  const int b = bh / a.H, h = bh - b * a.H;
  return b * a.Hkv + h / (a.H / a.Hkv);
}

__device__ __forceinline__ void work_item(const FwdArgs& a, int L, int& bh, int& qb) {
  const int nqb = a.nqb;
  if (a.order == kOrderHeavyFirst) {
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
