// Backward pass of the fused attention for bf16 inputs (gfx950): dQ, dK, dV from Q, K,
// V, O, dO and the forward pass's LSE, with the same masks and score modifiers.
//
// The page "FlashAttention 4: ... για LLMs" (el.linux-konsole.com), sections "Κύρια
// Συμπεράσματα" and "Συμβατότητα και τρέχουσα κατάσταση", names the backward pass as
// the piece FA4 still lacks.  It is the chain rule through the forward definition:
//   P = exp(s - LSE) (recomputed from Q, K and the saved LSE), dV = P^T dO,
//   dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D), dR = dS * ds/dr,
//   dQ = dR K, dK = dR^T Q   (ds/dr = scale, or scale * (1 - tanh^2) with softcap).
// Deterministic: no atomics.  Two launches:
//   dq_kernel    : one workgroup per (b*H + h, 128 query rows), a wave per 32 rows; it
//                  forms D of its rows (written for the second launch), then
//                  walks the row block's non-empty key blocks in 64-key steps:
//                  S^T = K Q^T and dP^T = V dO^T (Q and dO of the wave resident as
//                  B operands), dR^T elementwise, dQ^T += K^T dR^T.
//   dkdv_kernel  : one workgroup per (b*H_kv + g, 128 keys), a wave per 32 keys; it
//                  walks the query heads sharing the key/value head and their
//                  non-empty query blocks in 64-row steps: S = Q K^T and dP = dO V^T
//                  (K and V of the wave resident), dV^T += dO^T P, dK^T += Q^T dR.
// MFMA v_mfma_f32_32x32x16_bf16 throughout, with the forward pass's operand layouts:
// row fragments of a row-major LDS tile as A operands, transposed fragments
// (ds_read_b64_tr_b16) as A operands of the T^T products, and accumulators packed to
// bf16 as B operands in the contraction order those transposed reads produce.
#include <mutex>
#include <type_traits>

#include "../../include/attn119.h"

#include "common.hpp"

namespace attn119 {
namespace bwd {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef const __attribute__((address_space(4))) int cint;  // read-only, uniform: scalar loads
typedef const __attribute__((address_space(4))) unsigned char cu8;

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const bf16* dout;
  const float* lse;  // [B][H][N] natural log
  float* delta;      // [B][H][N] rowsum(dO * O)
  bf16* dq;
  bf16* dk;
  bf16* dv;
  int B, H, Hkv, N, nqb;
  float scale;
  float cap;        // softcap (flags & kSoftcap)
  float sc_cap;     // scale / cap
  float alibi_exp;  // default slopes 2^(alibi_exp (h+1)), alibi_exp = -8/H
  const float* alibi_slopes;
  uint32_t flags;   // every mask and modifier flag
  int window;
  const unsigned char* map;  // block map (positional masks)
  MapLayout lay;
  int compact;  // 1: the map is the compact form (a packed batch's workspace)
  int heavy;  // causal mask without documents: workgroups take the heaviest blocks first
};

// Order in which workgroups take their blocks (workgroup L runs on XCD L % 8).  Under a
// causal mask the work of a row block grows with its index and the work of a key block
// falls with it; in block order the long blocks would start last and leave most CUs idle
// at the end.  With `heavy` the blocks go out block-major, heaviest first (last row
// block first for dQ, first key block first for dK/dV), which is longest-first list
// scheduling; when the item's heads are a multiple of 8, XCD x takes the contiguous
// heads x*n/8 .. (x+1)*n/8-1, so the workgroups of one head share an L2.
__device__ __forceinline__ void bwd_item(int L, int nheads, int nblk, bool heavy, bool rising, int& head,
                                         int& blk) {
  if (heavy) {
    const int r = L / nheads, i = L - r * nheads;
    head = (nheads & 7) ? i : (i & 7) * (nheads >> 3) + (i >> 3);
    blk = rising ? r : nblk - 1 - r;
  } else {
    head = L / nblk;
    blk = L - head * nblk;
  }
}

constexpr float kLog2e = 1.4426950408889634f;
// LDS tiles: rows of 2D bytes, 16-byte chunk ch of row r stored at chunk position
// ch ^ lds_swz(r).  The tiles are read two ways: row fragments (16 lanes: 16 consecutive
// rows, one chunk) and transposed fragments (32 lanes: 4 consecutive rows, 4 consecutive
// chunks); lds_swz spreads both over 16 different 16-byte slots of a 256-byte line (d =
// 64: two rows per line), and the tile writes (8 lanes: 8 chunks of one row) over 8.  It
// depends on the row's low 4 bits only, so per-lane offsets survive 16-row steps.
template <int D>
__device__ __forceinline__ constexpr int lds_swz(int r) {
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ bf16x2 to_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_convertvector(v, bf16x2);
}
// registers 8g .. 8g+7 of an accumulator as a bf16 B operand
__device__ __forceinline__ bf16x8 pack8(const f32x16& acc, int g) {
  const bf16x2 a = to_bf16x2(acc[8 * g + 0], acc[8 * g + 1]), b = to_bf16x2(acc[8 * g + 2], acc[8 * g + 3]);
  const bf16x2 c = to_bf16x2(acc[8 * g + 4], acc[8 * g + 5]), d = to_bf16x2(acc[8 * g + 6], acc[8 * g + 7]);
  const u32x4 w = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                   __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// The same product with the register files chosen here, for the dK/dV kernel, whose
// accumulators, resident K and V and S/dP tiles need more than either file alone:
// acc += a b with acc in AGPRs, and d = a b / acc += a b with d, acc in VGPRs and b in
// AGPRs.  The compiler does not see these as MFMAs, so the code that uses them covers
// the hazards itself: a VALU read of an MFMA result waits kMfmaToValu wait states after
// the last MFMA that wrote it (an s_nop), and so does the epilogue's read of the AGPR
// accumulators; chained MFMAs on one accumulator (same opcode, same registers) and LDS
// loads into an operand (s_waitcnt, which the compiler inserts for asm operands too) need
// nothing more.
__device__ __forceinline__ void mfma_agpr(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v0(f32x16& d, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_v(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
// wait states between an 8-pass XDL op writing a register and a VALU op reading it, with
// margin (three s_nop 7: 24)
__device__ __forceinline__ void mfma_result_wait() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}
// row offset (minus 4*hh) of accumulator register r: 8*(r>>2) + (r&3)
__device__ __forceinline__ constexpr int acc_row(int r) { return 8 * (r >> 2) + (r & 3); }

// A fragment of a row-major tile (stride STR): row r0 + l32, 8 values at column 16c + 8hh
// (rsw = lds_swz(l32); r0 is a multiple of 32)
template <int STR>
__device__ __forceinline__ bf16x8 row_frag(const lds_u8* t, int r0, int l32, int hh, int c, int rsw) {
  return *(const lds_bf16x8*)(t + (r0 + l32) * STR + (((2 * c + hh) ^ rsw) << 4));
}
// A fragment of the transpose of a row-major tile: columns 32db .. 32db+31 as rows, the
// 16 tile rows 16ks .. 16ks+15 as k, in the order 4hh+e, 8+4hh+e (e = 0..3) that the
// accumulator registers 8g .. 8g+7 carry; off = this lane's offset for block db.
template <int STR>
__device__ __forceinline__ bf16x8 tr_frag(const lds_u8* t, int ks, int2 off) {
  const lds_u8* base = t + ks * 16 * STR;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off.x));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off.y));
  const short __attribute__((ext_vector_type(8))) w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, w);
}
// this lane's offsets (rows 4hh + e and 8 + 4hh + e of a 16-row group) for block db
template <int D>
__device__ __forceinline__ int2 tr_off(int lane, int db) {
  constexpr int STR = 2 * D;
  const int e = (lane & 15) >> 2, aa = lane & 3, dh = (lane >> 4) & 1, hh = lane >> 5;
  const int chunk = 4 * db + 2 * dh + (aa >> 1);
  const int r = 4 * hh + e;
  return make_int2(r * STR + ((chunk ^ lds_swz<D>(r)) << 4) + (aa & 1) * 8,
                   (r + 8) * STR + ((chunk ^ lds_swz<D>(r + 8)) << 4) + (aa & 1) * 8);
}

// Per-kernel constants of the score modifiers, folded for the log2 domain.
struct ScoreConsts {
  float sl2;    // scale * log2(e)
  float sce;    // 2 log2(e) scale / cap (softcap: exp2(raw sce) = e^(2 y), y = raw scale / cap)
  float capl2;  // cap * log2(e)
};
__device__ __forceinline__ ScoreConsts score_consts(const BwdArgs& a) {
  ScoreConsts c;
  c.sl2 = a.scale * kLog2e;
  c.sce = 2.f * kLog2e * a.sc_cap;
  c.capl2 = a.cap * kLog2e;
  return c;
}
// s log2(e) of one (q, k) element, and ds/dr divided by the scale (the scale is applied
// to dQ and dK once, at the end); the modifiers are template parameters, so there is no
// branch per element.  softcap: s = cap tanh(y), tanh(y) = 1 - 2 / (e^(2y) + 1),
// ds/dr = scale (1 - tanh^2); ALiBi: s -= slope |q - k| (slope2 = slope log2(e)).
template <bool SOFTCAP, bool ALIBI>
__device__ __forceinline__ float score2(const ScoreConsts& c, float raw, int q, int k, float slope2, float& dsdr) {
  float x;
  if constexpr (SOFTCAP) {
    const float t = 1.f - 2.f * rcp_(exp2_(raw * c.sce) + 1.f);
    dsdr = __builtin_fmaf(-t, t, 1.f);
    x = t * c.capl2;
  } else {
    x = raw * c.sl2;
  }
  if constexpr (ALIBI) x = __builtin_fmaf(-slope2, (float)(q > k ? q - k : k - q), x);
  return x;
}
// p = exp(s - LSE) of an element, x = s log2(e), lse2 = LSE log2(e); a hidden element
// takes exp2(-inf) = 0 (no branch)
template <bool MASK>
__device__ __forceinline__ float prob2(bool vis, float x, float lse2) {
  if constexpr (MASK) return exp2_(vis ? x - lse2 : -__builtin_inff());
  return exp2_(x - lse2);
}

__device__ __forceinline__ float head_slope(const BwdArgs& a, int h) {
  return a.alibi_slopes ? a.alibi_slopes[h] : exp2_(a.alibi_exp * (float)(h + 1));
}

// Causal and window masks without documents, when the call passes no map: the keys row q
// sees, [row_lo_of(q), row_hi_of(q)], and the rows that see key k, [col_lo_of(k),
// col_hi_of(k)], from the flags (the values the map's interval sections would hold)
__device__ __forceinline__ int row_lo_of(const BwdArgs& a, int q) {
  return (a.flags & kWindow) ? max(0, q - (a.window - 1)) : 0;
}
__device__ __forceinline__ int row_hi_of(const BwdArgs& a, int q) {
  return (a.flags & kCausal) ? q : ((a.flags & kWindow) ? min(a.N - 1, q + (a.window - 1)) : a.N - 1);
}
__device__ __forceinline__ int col_lo_of(const BwdArgs& a, int k) {
  return (a.flags & kCausal) ? k : ((a.flags & kWindow) ? max(0, k - (a.window - 1)) : 0);
}
__device__ __forceinline__ int col_hi_of(const BwdArgs& a, int k) {
  return (a.flags & kWindow) ? min(a.N - 1, k + (a.window - 1)) : a.N - 1;
}

// header of the block map matches the call, and (document masks) no batch row is
// marked invalid; uniform over the workgroup
__device__ bool map_invalid(const BwdArgs& a, int b) {
  const MapHeader* hd = (const MapHeader*)a.map;
  bool bad = hd->magic != kMapMagic || hd->B != a.B || hd->N != a.N || hd->flags != (a.flags & kPositional) ||
             hd->window != ((a.flags & kWindow) ? a.window : 0) || hd->compact != a.compact;
  int st = 0;
  if (a.flags & kDocument) {
    const int* s = (const int*)(a.map + a.lay.status) + (size_t)b * a.nqb;
    for (int i = threadIdx.x; i < a.nqb; i += 256) st |= s[i];
  }
  return __syncthreads_or(st) != 0 || bad;
}

// ---- dQ ----------------------------------------------------------------------------------
template <int D, bool MASKED, bool SOFTCAP, bool ALIBI>
__global__ void __launch_bounds__(256, 2) dq_kernel(const BwdArgs a) {
  constexpr int ROWB = 2 * D, STR = ROWB, CPR = ROWB / 16, NQC = D / 16, NDB = D / 32;
  constexpr int BN = 64;
  constexpr int TILE = BN * STR, LPW = TILE / 1024 / 4, RPL = 1024 / ROWB;  // 1 KiB direct loads
  // K and V tiles, double-buffered: step s reads buffer s % 2 while the tiles of step s+1
  // arrive in the other one straight from HBM
  __shared__ __attribute__((aligned(1024))) unsigned char k_sh[2][TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_sh[2][TILE];

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-wave choices stay scalar
  const int N = a.N, nqb = a.nqb;
  int bh, qb;
  bwd_item(blockIdx.x, a.B * a.H, nqb, a.heavy, false, bh, qb);
  const int b = bh / a.H, h = bh - b * a.H;
  const int bkv = b * a.Hkv + h / (a.H / a.Hkv);
  const int qrow = qb * 128 + wave * 32 + l32;
  const bool qvalid = qrow < N;
  const size_t qoff = ((size_t)bh * N + (qvalid ? qrow : 0)) * D;
  // direct HBM -> LDS loads: load r of this wave fills LDS bytes 1024 (wave LPW + r) +
  // 16 lane, i.e. row ld RPL + lane / CPR at chunk position lane % CPR, which holds the
  // row's chunk (position ^ lds_swz(row)); the buffer descriptor of a step starts at its
  // first key and ends at N, so rows past N read as zero
  int ldoff[LPW];
#pragma unroll
  for (int r = 0; r < LPW; ++r) {
    const int row = (wave * LPW + r) * RPL + lane / CPR, pc = lane % CPR;
    ldoff[r] = row * ROWB + ((pc ^ lds_swz<D>(row)) << 4);
  }
  const unsigned char* const kbase = (const unsigned char*)a.k + (size_t)bkv * N * ROWB;
  const unsigned char* const vbase = (const unsigned char*)a.v + (size_t)bkv * N * ROWB;
  // (untracked by the compiler: each step waits for its own tiles before its barrier)
  auto issue = [&](int k0, int buf) {
    const int bytes = max(N - k0, 0) * ROWB;
    const u32x4 krs = dma_rsrc(kbase + (size_t)k0 * ROWB, bytes);
    const u32x4 vrs = dma_rsrc(vbase + (size_t)k0 * ROWB, bytes);
#pragma unroll
    for (int r = 0; r < LPW; ++r) {
      dma_to_lds<16>(krs, (lds_u8*)k_sh[buf] + (wave * LPW + r) * 1024, ldoff[r]);
      dma_to_lds<16>(vrs, (lds_u8*)v_sh[buf] + (wave * LPW + r) * 1024, ldoff[r]);
    }
  };

  bf16x8 qf[NQC], gf[NQC];
#pragma unroll
  for (int c = 0; c < NQC; ++c) {
    qf[c] = qvalid ? *(const bf16x8*)(a.q + qoff + 16 * c + 8 * hh) : bf16x8{};
    gf[c] = qvalid ? *(const bf16x8*)(a.dout + qoff + 16 * c + 8 * hh) : bf16x8{};
  }
  const float lse2 = qvalid ? a.lse[(size_t)bh * N + qrow] * kLog2e : 0.f;
  const ScoreConsts mc = score_consts(a);
  // D = rowsum(dO * O) of the lane's row: the lane holds the dO values 16c + 8hh .. +7 of
  // the row, its partner lane (lane ^ 32) the others; the O values at the same places
  // are loaded beside them.  D is written here for the dK/dV kernel, launched after.
  float dl = 0.f;
#pragma unroll
  for (int c = 0; c < NQC; ++c) {
    const u32x4 ov = qvalid ? *(const u32x4*)(a.o + qoff + 16 * c + 8 * hh) : u32x4{0, 0, 0, 0};
    const u32x4 gv = __builtin_bit_cast(u32x4, gf[c]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      dl = __builtin_fmaf(__uint_as_float(ov[t] << 16), __uint_as_float(gv[t] << 16), dl);
      dl = __builtin_fmaf(__uint_as_float(ov[t] & 0xFFFF0000u), __uint_as_float(gv[t] & 0xFFFF0000u), dl);
    }
  }
  dl = pair_sum(dl);
  if (qvalid && hh == 0) a.delta[(size_t)bh * N + qrow] = dl;
  const float slope2 = ALIBI ? head_slope(a, h) * kLog2e : 0.f;

  int lo_q = 0, hi_q = qvalid ? N - 1 : -1;
  int nblk = nqb, npart = 0;
  // The key blocks of this query block, from the map's row intervals of its first and
  // last rows r0, r1 (every row sees [row_lo, row_hi], both ends non-decreasing, the row
  // itself inside): non-empty are ua .. ub, FULL fa .. fb (inside [lo(r1), hi(r0)], 128
  // rows and keys), PARTIAL the pl blocks left of the FULL range and those right of it;
  // step order: the PARTIAL blocks ascending, then the FULL ones (the map's lists are not
  // read).  Without a map (causal and window masks) the intervals follow from the flags.
  int ua = 0, fa = 0, fb = -1, pl = 0;
  bool invalid = false;
  if constexpr (MASKED) {
    const bool derive = a.map == nullptr;
    if (!derive) invalid = map_invalid(a, b);
    {
      const int r0 = qb * 128, r1 = min(N, r0 + 128) - 1;
      int lo0, lo1, hi0, hi1;
      if (derive) {
        lo0 = row_lo_of(a, r0);
        lo1 = row_lo_of(a, r1);
        hi0 = row_hi_of(a, r0);
        hi1 = row_hi_of(a, r1);
      } else {
        typedef const __attribute__((address_space(4))) int cint4;
        cint4* rlo = (cint4*)(a.map + a.lay.row_lo) + (size_t)b * N;
        cint4* rhi = (cint4*)(a.map + a.lay.row_hi) + (size_t)b * N;
        lo0 = rlo[r0];
        lo1 = rlo[r1];
        hi0 = rhi[r0];
        hi1 = rhi[r1];
      }
      ua = min(max(lo0 >> 7, 0), nqb - 1);
      const int ub = hi1 < lo0 ? ua - 1 : min(hi1 >> 7, nqb - 1);
      fa = max(ua, (lo1 + 127) >> 7);
      fb = min(ub, ((hi0 + 1) >> 7) - 1);
      if (r1 - r0 != 127 || fa > fb) { fa = ub + 1; fb = ub; }  // no FULL block
      const int nfull = fb - fa + 1;
      npart = max(ub - ua + 1 - nfull, 0);
      pl = fa - ua;
      nblk = invalid ? 0 : nfull + npart;
    }
    if (qvalid) {
      lo_q = derive ? row_lo_of(a, qrow) : ((const int*)(a.map + a.lay.row_lo))[(size_t)b * N + qrow];
      hi_q = derive ? row_hi_of(a, qrow) : ((const int*)(a.map + a.lay.row_hi))[(size_t)b * N + qrow];
    }
  }
  int2 troff[NDB];
  const int rsw = lds_swz<D>(l32);
#pragma unroll
  for (int db = 0; db < NDB; ++db) troff[db] = tr_off<D>(lane, db);

  f32x16 dacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dacc[db] = f32x16{};

  // Steps s = 0 .. 2*nblk-1 (64 keys each).  The tiles of step s+1 are requested into the
  // other LDS buffer as step s starts; one barrier per step.
  auto step_k0 = [&](int st_) -> int {
    int kb = st_ >> 1;
    if constexpr (MASKED) {
      const int i = st_ >> 1;
      kb = i < pl ? ua + i : (i < npart ? fb + 1 + (i - pl) : fa + (i - npart));
      kb = min(max(kb, 0), nqb - 1);
    }
    return kb * 128 + (st_ & 1) * BN;
  };
  const int nsteps = 2 * nblk;
  if (nsteps > 0) issue(step_k0(0), 0);
  // (the wave's Q, dO rows and per-row values, loaded above, have arrived: a wait the
  // compiler sees, so that it puts none for them inside the loops)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // one step; the PARTIAL blocks' steps come first (with the mask), then the FULL ones,
  // each kind in a loop of its own
  auto step = [&](const int st_, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k0 = step_k0(st_);
    // this wave's loads of step st_ have landed; after the barrier every wave's have, and
    // every wave is done reading the buffer the next loads go to (step st_ - 1)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (st_ + 1 < nsteps) issue(step_k0(st_ + 1), (st_ + 1) & 1);
    const lds_u8* kt = (const lds_u8*)k_sh[st_ & 1];
    const lds_u8* vt = (const lds_u8*)v_sh[st_ & 1];
    // The step as one stream of MFMA slots: S^T and dP^T of keys 0-31 (SP0), of keys 32-63
    // (SP1), then dQ^T from keys 0-31 (DQ0) and from keys 32-63 (DQ1).  Every slot reads
    // its LDS fragment PD slots ahead; dR^T of keys 0-31 is formed on the vector ALU under
    // SP1, of keys 32-63 under DQ0; scheduling fences keep the slots in this order.  A FULL
    // block (and every step without a positional mask: keys past N are zero rows of K and
    // V, so they add nothing to dQ) needs no mask.
    constexpr int NSP = 2 * NQC, NDQ = 2 * NDB, NM = 2 * (NSP + NDQ), PD = 3;
    auto frag = [&](auto ic) -> bf16x8 {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < 2 * NSP) {
        constexpr int bk = i / NSP, c = (i % NSP) / 2;
        return row_frag<STR>((i & 1) ? vt : kt, 32 * bk, l32, hh, c, rsw);
      } else {
        constexpr int t = i - 2 * NSP, ks = t / NDB, db = t % NDB;
        return tr_frag<STR>(kt, ks, troff[db]);
      }
    };
    {
      f32x16 st[2], dp[2];
      bf16x8 bop[4];
      // dR^T of accumulator register r of key slice bk
      auto elem = [&](int bk, int r) {
        const int key = k0 + 32 * bk + 4 * hh + acc_row(r);
        float dsdr = 1.f;
        const float x = score2<SOFTCAP, ALIBI>(mc, st[bk][r], qrow, key, slope2, dsdr);
        const float p = prob2<MASK>(key >= lo_q && key <= hi_q, x, lse2);
        const float g = p * (dp[bk][r] - dl);
        st[bk][r] = SOFTCAP ? g * dsdr : g;
      };
      // elementwise work of slot k of a phase of n slots, and the bf16 operands of a
      // half once its 8 registers are done
      auto elems = [&](int bk, int k, int n) {
        const int r0 = 16 * k / n, r1 = 16 * (k + 1) / n;
        for (int r = r0; r < r1; ++r) elem(bk, r);
        if (r0 < 8 && r1 >= 8) bop[2 * bk] = pack8(st[bk], 0);
        if (r1 == 16) bop[2 * bk + 1] = pack8(st[bk], 1);
      };
      bf16x8 fr[PD + 1];
      static_for<PD>([&](auto ic) { fr[ic.value] = frag(ic); });
      st[0] = st[1] = dp[0] = dp[1] = f32x16{};
      __builtin_amdgcn_sched_barrier(0);
      static_for<NM>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + PD < NM) fr[(i + PD) % (PD + 1)] = frag(std::integral_constant<int, i + PD>{});
        const bf16x8 f = fr[i % (PD + 1)];
        if constexpr (i < 2 * NSP) {
          constexpr int bk = i / NSP, c = (i % NSP) / 2, k = i % NSP;
          if constexpr (i & 1)
            dp[bk] = mfma(f, gf[c], dp[bk]);
          else
            st[bk] = mfma(f, qf[c], st[bk]);
          if constexpr (bk == 1) elems(0, k, NSP);
        } else {
          constexpr int t = i - 2 * NSP, ks = t / NDB, db = t % NDB;
          dacc[db] = mfma(f, bop[ks], dacc[db]);
          if constexpr (t < NDQ) elems(1, t, NDQ);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    }
  };
  int st_ = 0;
  if constexpr (MASKED)
    for (; st_ < 2 * npart; ++st_) step(st_, std::true_type{});
  for (; st_ < nsteps; ++st_) step(st_, std::false_type{});
  if (!qvalid) return;
  const float nanv = __builtin_bit_cast(float, 0x7fc00000u);
  bf16* dst = a.dq + qoff;
#pragma unroll
  for (int db = 0; db < NDB; ++db) dacc[db] *= a.scale;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x16& x = dacc[db];
      const bf16x2 v01 = invalid ? to_bf16x2(nanv, nanv) : to_bf16x2(x[4 * i], x[4 * i + 1]);
      const bf16x2 v23 = invalid ? to_bf16x2(nanv, nanv) : to_bf16x2(x[4 * i + 2], x[4 * i + 3]);
      const u32x2 w = {__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23)};
      *(u32x2*)(dst + db * 32 + 8 * i + 4 * hh) = w;
    }
}

// ---- dK, dV ------------------------------------------------------------------------------
template <int D, bool MASKED, bool SOFTCAP, bool ALIBI>
__global__ void __launch_bounds__(256, 1) dkdv_kernel(const BwdArgs a) {
  constexpr int ROWB = 2 * D, STR = ROWB, CPR = ROWB / 16, NQC = D / 16, NDB = D / 32;
  constexpr int BM = 64;  // query rows per step
  constexpr int NBQ = BM / 32;
  constexpr int TILE = BM * STR, LPW = TILE / 1024 / 4, RPL = 1024 / ROWB;  // 1 KiB direct loads
  static_assert(LPW == 4 || LPW == 2, "the step-top wait counts 2 LPW tile loads");
  // Q and dO tiles of a step in three buffers: step s reads buffer s % 3 while the rows of
  // steps s+1 and s+2 arrive in the other two straight from HBM (two steps of latency
  // cover); the per-row values likewise
  constexpr int NBUF = 3;
  __shared__ __attribute__((aligned(1024))) unsigned char q_sh[NBUF][TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char g_sh[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) float lse_s[NBUF][BM];
  __shared__ __attribute__((aligned(16))) float dl_s[NBUF][BM];
  __shared__ __attribute__((aligned(16))) int lo_s[NBUF][BM];
  __shared__ __attribute__((aligned(16))) int hi_s[NBUF][BM];

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-wave choices stay scalar
  const int N = a.N, nqb = a.nqb;
  int bkv, kb;
  bwd_item(blockIdx.x, a.B * a.Hkv, nqb, a.heavy, true, bkv, kb);
  const int b = bkv / a.Hkv, kvh = bkv - b * a.Hkv;
  const int grp = a.H / a.Hkv;
  const int key = kb * 128 + wave * 32 + l32;
  const bool kvalid = key < N;
  const size_t koff = ((size_t)bkv * N + (kvalid ? key : 0)) * D;

  bf16x8 kf[NQC], vf[NQC];
#pragma unroll
  for (int c = 0; c < NQC; ++c) {
    kf[c] = kvalid ? *(const bf16x8*)(a.k + koff + 16 * c + 8 * hh) : bf16x8{};
    vf[c] = kvalid ? *(const bf16x8*)(a.v + koff + 16 * c + 8 * hh) : bf16x8{};
  }
  bool invalid = false;
  const bool derive = MASKED && a.map == nullptr;  // causal and window masks without a map
  if constexpr (MASKED) {
    if (!derive) invalid = map_invalid(a, b);
  }
  int2 troff[NDB];
  const int rsw = lds_swz<D>(l32);
#pragma unroll
  for (int db = 0; db < NDB; ++db) troff[db] = tr_off<D>(lane, db);

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }
  const ScoreConsts mc = score_consts(a);
  // The query blocks this key block is visible from, from the map's column intervals: the
  // rows that see key k are [col_lo(k), col_hi(k)], both ends non-decreasing in k and k
  // itself inside (every mask here), so the rows that see some key of the block form the
  // one range [col_lo(k0), col_hi(k1)] of its first and last keys k0, k1 -- non-empty
  // query blocks qa .. qz -- and a query block is FULL (every row sees every key) when it
  // lies in [col_lo(k1), col_hi(k0)] with 128 rows, and the key block has 128 keys.  (The
  // same argument as the forward pass's, with rows and keys swapped; the map's class and
  // list sections are not read.)
  int qa = 0, qz = nqb - 1, qfa = 0, qfz = nqb - 1;
  if constexpr (MASKED) {
    const int k0 = kb * 128, k1 = min(N, k0 + 128) - 1;
    int lo0, lo1, hi0, hi1;
    if (derive) {
      lo0 = col_lo_of(a, k0);
      lo1 = col_lo_of(a, k1);
      hi0 = col_hi_of(a, k0);
      hi1 = col_hi_of(a, k1);
    } else {
      typedef const __attribute__((address_space(4))) int cint4;
      cint4* clo = (cint4*)(a.map + a.lay.col_lo) + (size_t)b * N;
      cint4* chi = (cint4*)(a.map + a.lay.col_hi) + (size_t)b * N;
      lo0 = clo[k0];
      lo1 = clo[k1];
      hi0 = chi[k0];
      hi1 = chi[k1];
    }
    qa = min(max(lo0 >> 7, 0), nqb);
    qz = hi1 < lo0 ? -1 : min(hi1 >> 7, nqb - 1);
    qfa = max(qa, (lo1 + 127) >> 7);
    qfz = min(qz, ((hi0 + 1) >> 7) - 1);
    if (k1 - k0 != 127) qfz = qfa - 1;  // a key block cut by N is never FULL
  }
  // class of query block qb (in qa .. qz) against this key block: 2 FULL, 1 PARTIAL
  auto cls_of = [&](int qb) -> int { return (qb >= qfa) & (qb <= qfz) ? 2 : 1; };
  // first non-empty query block at or after `from` (nqb if none)
  auto next_block = [&](int from) -> int {
    if constexpr (!MASKED) return from;
    const int q = max(from, qa);
    return q <= qz ? q : nqb;
  };
  // Steps: (query head of the group, non-empty query block, 64-row sub-block), in that
  // nesting.  next() advances a step state.
  auto next = [&](int& hq, int& qb, int& sub) -> bool {
    ++sub;
    if (sub == 128 / BM || qb * 128 + sub * BM >= N) {
      sub = 0;
      for (;;) {
        qb = next_block(qb + 1);
        if (qb < nqb) break;
        qb = -1;
        if (++hq == grp) return false;
      }
    }
    return true;
  };
  // direct HBM -> LDS loads (the layout of the dQ kernel's): load r of this wave fills LDS
  // bytes 1024 (wave LPW + r) + 16 lane, row ld RPL + lane / CPR at chunk position lane %
  // CPR, which holds the row's chunk (position ^ lds_swz(row)); the buffer descriptor of a
  // step starts at its first row and ends at N, so rows past N read as zero
  int ldoff[LPW];
#pragma unroll
  for (int r = 0; r < LPW; ++r) {
    const int row = (wave * LPW + r) * RPL + lane / CPR, pc = lane % CPR;
    ldoff[r] = row * ROWB + ((pc ^ lds_swz<D>(row)) << 4);
  }
  // Requests a step's Q and dO rows into buffer buf, and its per-row values into the
  // per-row arrays: one 256-byte load per wave (wave 0: the LSE, 1: D, 2 and 3: the first
  // and last visible key; without a positional mask waves 2 and 3 load the LSE and D
  // again into the interval arrays, which nothing reads; with a positional mask but no
  // map waves 2 and 3 load them into arrays of their own that nothing reads, and write
  // the intervals from the flags), so every wave has 2 LPW + 1 loads in flight per step.
  // Rows past N read as zero (Q, dO, LSE, D and the interval [0, 0]): such a row adds
  // nothing to any gradient.
  constexpr int LPS = 2 * LPW + 1;
  __shared__ __attribute__((aligned(16))) int unread_s[2][NBUF][BM];
  auto fetch = [&](int hq, int qb, int sub, int buf) {
    const int bh = b * a.H + kvh * grp + hq;
    const int q0 = qb * 128 + sub * BM;
    const int rows = max(N - q0, 0);
    const float* lse_src = a.lse + (size_t)bh * N + q0;
    const float* dl_src = a.delta + (size_t)bh * N + q0;
    const void* src = (wave & 1) ? (const void*)dl_src : (const void*)lse_src;
    if constexpr (MASKED) {
      if (wave >= 2 && !derive)
        src = (const int*)(a.map + ((wave & 1) ? a.lay.row_hi : a.lay.row_lo)) + (size_t)b * N + q0;
    }
    lds_u8* dst = wave == 0 ? (lds_u8*)lse_s[buf] : wave == 1 ? (lds_u8*)dl_s[buf]
                : wave == 2 ? (lds_u8*)lo_s[buf] : (lds_u8*)hi_s[buf];
    if (derive && wave >= 2) dst = (lds_u8*)unread_s[wave & 1][buf];
    dma_to_lds<4>(dma_rsrc(src, rows * 4), dst, 4 * lane);
    if (derive && wave >= 2) {  // row q0 + lane of the step (BM = 64 rows, one per lane)
      const int q = q0 + lane;
      const int v = q < N ? ((wave & 1) ? row_hi_of(a, q) : row_lo_of(a, q)) : 0;
      ((wave & 1) ? hi_s[buf] : lo_s[buf])[lane] = v;
    }
    const int bytes = rows * ROWB;
    const u32x4 qrs = dma_rsrc((const unsigned char*)a.q + ((size_t)bh * N + q0) * ROWB, bytes);
    const u32x4 grs = dma_rsrc((const unsigned char*)a.dout + ((size_t)bh * N + q0) * ROWB, bytes);
#pragma unroll
    for (int r = 0; r < LPW; ++r) {
      dma_to_lds<16>(qrs, (lds_u8*)q_sh[buf] + (wave * LPW + r) * 1024, ldoff[r]);
      dma_to_lds<16>(grs, (lds_u8*)g_sh[buf] + (wave * LPW + r) * 1024, ldoff[r]);
    }
  };
  // the current step (hq, qb, sub) and the two after it
  int hq = 0, qb = -1, sub = 128 / BM - 1;
  bool have = !invalid && next(hq, qb, sub);
  int h1 = hq, q1 = qb, s1 = sub;
  bool have1 = have && next(h1, q1, s1);
  if (have) fetch(hq, qb, sub, 0);
  if (have1) fetch(h1, q1, s1, 1);
  int buf = 0;
  // (K and V of the wave, loaded above, have arrived: a wait the compiler sees, so that it
  // puts no wait for them inside the loop, where its count would include the tile loads)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  static_assert(LPS == 9 || LPS == 5, "the step-top wait below counts LPS loads");
  while (have) {
    const int h = kvh * grp + hq;
    const int q0 = qb * 128 + sub * BM;
    const float slope2 = ALIBI ? head_slope(a, h) * kLog2e : 0.f;
    // this wave's loads of the step have landed (only the LPS of the next step may still
    // be in flight: the loads complete in order); after the barrier every wave's have, and
    // every wave is done reading the buffers of step - 1, which the loads of step + 2 go to
    if (have1) {
      if constexpr (LPS == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    int h2 = h1, q2 = q1, s2 = s1;
    const bool have2 = have1 && next(h2, q2, s2);
    const int buf2 = buf >= NBUF - 2 ? buf + 2 - NBUF : buf + 2;
    if (have2) fetch(h2, q2, s2, buf2);
    const lds_u8* qt = (const lds_u8*)q_sh[buf];
    const lds_u8* gt = (const lds_u8*)g_sh[buf];
    const float* lse_b = lse_s[buf];
    const float* dl_b = dl_s[buf];
    const int* lo_b = lo_s[buf];
    const int* hi_b = hi_s[buf];
    // The step as one stream of MFMA slots, in this order: S and dP of rows 0-31 (SP0),
    // of rows 32-63 (SP1), then dV and dK from rows 0-31 (TR0) and from rows 32-63 (TR1).
    // Every slot reads its LDS fragment PD slots ahead, and the elementwise work of a
    // 32-row slice runs on the vector ALU under the MFMAs of the next phase: P and dR of
    // rows 0-31 under SP1, of rows 32-63 under TR0, each group of 4 rows' values read
    // from LDS RA slots before its first use.  Scheduling fences keep the slots in this
    // order.  Every step of a kernel with a positional mask applies the rows' key intervals
    // (a FULL block's hold every key of it; a second, unmasked body for FULL blocks made
    // the register allocator shuttle the accumulators between the register files every
    // step); without one every element is visible (rows and keys past N are zero rows of
    // Q, dO, K and V, so they add nothing to any gradient).
    static_assert(NBQ == 2, "two 32-row slices per step");
    constexpr int NSP = 2 * NQC, NTR = 4 * NDB, NM = 2 * (NSP + NTR), PD = 4, RA = 4;
    auto frag = [&](auto ic) -> bf16x8 {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < 2 * NSP) {
        constexpr int bq = i / NSP, c = (i % NSP) / 2;
        return row_frag<STR>((i & 1) ? gt : qt, 32 * bq, l32, hh, c, rsw);
      } else {
        constexpr int t = i - 2 * NSP, bq = t / NTR, g = (t % NTR) / (2 * NDB), db = (t % (2 * NDB)) / 2;
        return tr_frag<STR>((t & 1) ? qt : gt, 2 * bq + g, troff[db]);
      }
    };
    // Without softcap the mask can ride on the S accumulators: S starts as a bias of 0 where
    // the row sees the lane's key and -inf where it does not, so a hidden score stays -inf
    // through the products and the ALiBi term and its p is 0 -- and only the steps of
    // PARTIAL blocks compute the bias (FULL blocks start S at 0).  With softcap a hidden
    // score would come out finite (tanh saturates), so there the elementwise stage applies
    // the mask in every step.
    constexpr bool BIAS = MASKED && !SOFTCAP;
    auto run = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      // per-row values of slice bq, rows 32bq + 8j + 4hh .. +3 (one 16-byte LDS read each)
      float4 rl[2][4], rd[2][4];
      int4 rlo[2][4], rhi[2][4];
      auto read_rows = [&](int bq, int j) {
        const int q4 = 32 * bq + 4 * hh + 8 * j;
        rl[bq][j] = *(const float4*)&lse_b[q4] * kLog2e;
        rd[bq][j] = *(const float4*)&dl_b[q4];
        if constexpr (MASK) {
          rlo[bq][j] = *(const int4*)&lo_b[q4];
          rhi[bq][j] = *(const int4*)&hi_b[q4];
        }
      };
      f32x16 s[2], dp[2];
      u32x4 pbw[2][2], rbw[2][2];  // bf16 pairs of P and dR: word w of half g = registers 8g + 2w, +1
      // The elementwise work of an element (accumulator register r of slice bq: row
      // 32bq + 8(r/4) + 4hh + r%4) in NSTG stages, stage st in the slot st after the
      // element's entry slot: the slots then carry stages of NSTG different elements,
      // whose independent chains hide each other's latency (one element per slot, start to
      // finish, left the vector ALU waiting on each result in turn).
      //   linear scores: x = s log2 e (ALiBi bias), g = dP - D | arg | p = exp2(arg) | P, dR
      //   softcap:       e = exp2(2y), g | r = rcp(e + 1) | t = 1 - 2r, x, ds/dr, arg |
      //                  p = exp2(arg) | P, dR
      constexpr int NSTG = SOFTCAP ? 5 : 4;
      float eu[2][16], eg[2][16], ed[2][16], ep[2][16], em[2][16];
      auto stage = [&](auto stc, int bq, int r) {
        constexpr int st = decltype(stc)::value;
        const int j = r >> 2, e = r & 3;
        const int q = q0 + 32 * bq + 8 * j + 4 * hh + e;
        auto alibi = [&](float x) {
          if constexpr (ALIBI) x = __builtin_fmaf(-slope2, (float)(q > key ? q - key : key - q), x);
          return x;
        };
        auto arg_of = [&](float x) {
          const float ls = rl[bq][j][e];
          if constexpr (MASK) return ((key >= rlo[bq][j][e]) & (key <= rhi[bq][j][e])) ? x - ls : -__builtin_inff();
          return x - ls;
        };
        if constexpr (st == 0) {
          eg[bq][r] = dp[bq][r] - rd[bq][j][e];
          if constexpr (SOFTCAP) eu[bq][r] = exp2_(s[bq][r] * mc.sce);
          else if constexpr (!ALIBI) eu[bq][r] = __builtin_fmaf(s[bq][r], mc.sl2, -rl[bq][j][e]);  // x - lse2
          else eu[bq][r] = alibi(s[bq][r] * mc.sl2);
        } else if constexpr (SOFTCAP && st == 1) {
          eu[bq][r] = rcp_(eu[bq][r] + 1.f);
        } else if constexpr (SOFTCAP && st == 2) {
          const float t = __builtin_fmaf(-2.f, eu[bq][r], 1.f);
          ed[bq][r] = __builtin_fmaf(-t, t, 1.f);
          ep[bq][r] = arg_of(alibi(t * mc.capl2));
        } else if constexpr (!SOFTCAP && st == 1) {
          if constexpr (ALIBI) {
            ep[bq][r] = arg_of(eu[bq][r]);
          } else {  // (eu already holds x - lse2)
            if constexpr (MASK) ep[bq][r] = ((key >= rlo[bq][j][e]) & (key <= rhi[bq][j][e])) ? eu[bq][r] : -__builtin_inff();
            else ep[bq][r] = eu[bq][r];
          }
        } else if constexpr (st == NSTG - 2) {
          ep[bq][r] = exp2_(ep[bq][r]);
        } else if constexpr (st == NSTG - 1) {
          const float p = ep[bq][r];
          const float g = p * eg[bq][r];
          em[bq][r] = SOFTCAP ? g * ed[bq][r] : g;
          if (r & 1) {
            pbw[bq][r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, to_bf16x2(ep[bq][r - 1], p));
            rbw[bq][r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, to_bf16x2(em[bq][r - 1], em[bq][r]));
          }
        }
      };
      // elements of slice 0 enter under SP1, those of slice 1 under TR0, 16 / n per slot of
      // a phase of n slots; entry(bq, r) is the global slot of element r's first stage
      auto entry = [](int bq, int r) { return bq == 0 ? NSP + r / (16 / NSP) : 2 * NSP + r / (16 / NTR); };
      // (the last stage of every element of a half ends before the first MFMA that reads
      // the half: checked here for both slices and both halves)
      static_assert(entry(0, 7) + NSTG - 1 < 2 * NSP && entry(0, 15) + NSTG - 1 < 2 * NSP + 2 * NDB,
                    "P, dR of rows 0-31 are ready before their MFMAs");
      static_assert(entry(1, 7) + NSTG - 1 < 2 * NSP + NTR && entry(1, 15) + NSTG - 1 < 2 * NSP + NTR + 2 * NDB,
                    "P, dR of rows 32-63 are ready before their MFMAs");
      if constexpr (BIAS) {
        if (cls_of(qb) != 2) {  // a PARTIAL block: the rows' key intervals
#pragma unroll
          for (int bq = 0; bq < 2; ++bq)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int q4 = 32 * bq + 4 * hh + 8 * j;
              const int4 lo = *(const int4*)&lo_b[q4], hi = *(const int4*)&hi_b[q4];
              const int los[4] = {lo.x, lo.y, lo.z, lo.w}, his[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const bool vis = (key >= los[e]) & (key <= his[e]);  // (both compares, no branch)
                s[bq][4 * j + e] = vis ? 0.f : -__builtin_inff();
              }
            }
        } else {
          s[0] = f32x16{};
          s[1] = f32x16{};
        }
        // (a VALU write of a register an MFMA then reads as its accumulator needs wait
        // states the compiler does not add for these asm MFMAs)
        asm volatile("s_nop 7" ::: "memory");
      }
      bf16x8 fr[PD + 1];
      static_for<PD>([&](auto ic) { fr[ic.value] = frag(ic); });
      __builtin_amdgcn_sched_barrier(0);
      static_for<NM>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + PD < NM) fr[(i + PD) % (PD + 1)] = frag(std::integral_constant<int, i + PD>{});
        const bf16x8 f = fr[i % (PD + 1)];
        if constexpr (i < 2 * NSP) {
          constexpr int bq = i / NSP, c = (i % NSP) / 2, k = i % NSP;
          if constexpr (c == 0) {
            if constexpr (i & 1)
              mfma_v0(dp[bq], f, vf[c]);
            else if constexpr (BIAS)
              mfma_v(s[bq], f, kf[c]);  // onto the bias
            else
              mfma_v0(s[bq], f, kf[c]);
          } else {
            if constexpr (i & 1)
              mfma_v(dp[bq], f, vf[c]);
            else
              mfma_v(s[bq], f, kf[c]);
          }
          if constexpr (bq == 1 && k == 0) {
            mfma_result_wait();  // S, dP of rows 0-31 were written in the last two slots
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          constexpr int t = i - 2 * NSP, bq = t / NTR, g = (t % NTR) / (2 * NDB), db = (t % (2 * NDB)) / 2;
          if constexpr (t & 1)
            mfma_agpr(dkacc[db], f, __builtin_bit_cast(bf16x8, rbw[bq][g]));
          else
            mfma_agpr(dvacc[db], f, __builtin_bit_cast(bf16x8, pbw[bq][g]));
          if constexpr (t == 0) {
            mfma_result_wait();  // S, dP of rows 32-63 were written in the last two SP slots
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // the elementwise stages that fall in this slot (oldest element first): stage st of
        // the elements that entered in slot i - st
        static_for<NSTG>([&](auto sc) {
          constexpr int st = NSTG - 1 - decltype(sc)::value;
          static_for<2>([&](auto bc) {
            constexpr int bq = decltype(bc)::value, n = bq == 0 ? NSP : NTR, per = 16 / n;
            constexpr int k = i - st - (bq == 0 ? NSP : 2 * NSP);  // entry slot within the phase
            if constexpr (k >= 0 && k < n) {
              static_for<per>([&](auto uc) {
                constexpr int r = k * per + decltype(uc)::value;
                static_assert(entry(bq, r) == i - st, "entry slot");
                stage(std::integral_constant<int, st>{}, bq, r);
              });
            }
          });
        });
        // row group j of slice 0 is first used at slot NSP + j NSP / 4, of slice 1 at
        // slot 2 NSP + j NTR / 4
        static_for<4>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          if constexpr (i == NSP + j * NSP / 4 - RA) read_rows(0, j);
          if constexpr (i == 2 * NSP + j * NTR / 4 - RA) read_rows(1, j);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    run(std::bool_constant<MASKED && !BIAS>{});
    buf = buf == NBUF - 1 ? 0 : buf + 1;
    hq = h1;
    qb = q1;
    sub = s1;
    have = have1;
    h1 = h2;
    q1 = q2;
    s1 = s2;
    have1 = have2;
  }
  // (the accumulators leave the loop in AGPRs; without this pin the allocator copies them
  // to VGPRs at the loop head for the epilogue, and back before the MFMAs, every step)
#pragma unroll
  for (int db = 0; db < NDB; ++db) asm volatile("" : "+a"(dkacc[db]), "+a"(dvacc[db]));
  mfma_result_wait();  // the last step's MFMAs wrote the accumulators
  if (!kvalid) return;
  const float nanv = __builtin_bit_cast(float, 0x7fc00000u);
#pragma unroll
  for (int db = 0; db < NDB; ++db) dkacc[db] *= a.scale;
  bf16* dk = a.dk + koff;
  bf16* dv = a.dv + koff;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x16& x = dkacc[db];
      const f32x16& y = dvacc[db];
      const bf16x2 k01 = invalid ? to_bf16x2(nanv, nanv) : to_bf16x2(x[4 * i], x[4 * i + 1]);
      const bf16x2 k23 = invalid ? to_bf16x2(nanv, nanv) : to_bf16x2(x[4 * i + 2], x[4 * i + 3]);
      const bf16x2 v01 = invalid ? to_bf16x2(nanv, nanv) : to_bf16x2(y[4 * i], y[4 * i + 1]);
      const bf16x2 v23 = invalid ? to_bf16x2(nanv, nanv) : to_bf16x2(y[4 * i + 2], y[4 * i + 3]);
      *(u32x2*)(dk + db * 32 + 8 * i + 4 * hh) = u32x2{__builtin_bit_cast(uint32_t, k01), __builtin_bit_cast(uint32_t, k23)};
      *(u32x2*)(dv + db * 32 + 8 * i + 4 * hh) = u32x2{__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23)};
    }
}

template <int D, bool MASKED, bool SOFTCAP, bool ALIBI>
void launch_v(const BwdArgs& a, hipStream_t st) {
  const dim3 gq((unsigned)(a.B * a.H * a.nqb)), gk((unsigned)(a.B * a.Hkv * a.nqb)), blk(256);
  hipLaunchKernelGGL((dq_kernel<D, MASKED, SOFTCAP, ALIBI>), gq, blk, 0, st, a);
  hipLaunchKernelGGL((dkdv_kernel<D, MASKED, SOFTCAP, ALIBI>), gk, blk, 0, st, a);
}
template <int D, bool MASKED>
void launch_m(const BwdArgs& a, hipStream_t st) {
  const bool sc = a.flags & kSoftcap, al = a.flags & kAlibi;
  if (sc && al) launch_v<D, MASKED, true, true>(a, st);
  else if (sc) launch_v<D, MASKED, true, false>(a, st);
  else if (al) launch_v<D, MASKED, false, true>(a, st);
  else launch_v<D, MASKED, false, false>(a, st);
}
template <int D>
hipError_t launch_d(const BwdArgs& a, bool masked, hipStream_t st) {
  if (masked) launch_m<D, true>(a, st);
  else launch_m<D, false>(a, st);
  return hipGetLastError();
}

}  // namespace bwd

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv, float* delta, int B, int H, int Hkv, int N, int d, float scale,
                      uint32_t flags, int window, float softcap, const float* slopes, const void* map,
                      hipStream_t stream, bool compact_map) {
  bwd::BwdArgs a;
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.o = (const bf16*)o;
  a.dout = (const bf16*)dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = (bf16*)dq;
  a.dk = (bf16*)dk;
  a.dv = (bf16*)dv;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.nqb = (N + 127) / 128;
  a.scale = scale;
  a.cap = softcap;
  a.sc_cap = (flags & kSoftcap) ? (float)((double)scale / (double)softcap) : 0.f;
  a.alibi_exp = (float)(-8.0 / (double)H);
  a.alibi_slopes = slopes;
  a.flags = flags;
  a.window = window;
  a.map = (const unsigned char*)map;
  a.lay = map_layout(B, N, compact_map);
  a.compact = compact_map ? 1 : 0;
  a.heavy = (flags & kCausal) && !(flags & kDocument);
  const bool masked = (flags & kPositional) != 0;
  if (masked && !map && (flags & kDocument)) return hipErrorInvalidValue;  // (causal/window: derived)
  return d == 128 ? bwd::launch_d<128>(a, masked, stream) : bwd::launch_d<64>(a, masked, stream);
}

// ---- the backward pass without a caller workspace ------------------------------------
// For callers that cannot allocate (HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): the row sums D live in this file-scope device array instead of a
// caller-owned buffer.  Each GPU holds its own copy at its own address until the process
// ends; host code never passes the array's name (a host-side stand-in) to a kernel, only
// the device address hipGetSymbolAddress returns for the current device, looked up once
// per device.  Every call on a GPU shares that GPU's array, so calls that overlap on one
// GPU race; D is fully written by the dQ kernel before the dK/dV kernel reads it, so
// nothing needs clearing.
constexpr size_t kScratchRows = size_t(1) << 22;  // 4,194,304 rows of D = 16 MiB per GPU
static __device__ __align__(256) float scratch[kScratchRows];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t bwd_scratch_rows() { return kScratchRows; }

// Device address of this GPU's scratch array (resolved on the first call on the device).
hipError_t bwd_scratch_ptr(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                              float scale, uint32_t flags, int window, float softcap, const float* slopes,
                              const void* map, hipStream_t stream, bool compact_map) {
  if ((size_t)B * H * N > kScratchRows) return hipErrorInvalidValue;
  float* delta = nullptr;
  const hipError_t e = bwd_scratch_ptr(&delta);
  if (e != hipSuccess) return e;
  return launch_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hkv, N, d, scale, flags, window, softcap,
                    slopes, map, stream, compact_map);
}

}  // namespace attn119
