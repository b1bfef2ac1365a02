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
};

}  // namespace attn119
