// Fused, tiled exact-attention forward pass for gfx950 (MI355X).
//
// What is computed (pages, by title and section):
//  * "FlashAttention 4: Γρηγορότερη και Αποδοτική σε Μνήμη Προσοχή για LLMs"
//    (el.linux-konsole.com), "Εισαγωγή": scores Q.K^T, softmax, times V; only a
//    few rows of Q x K live on chip at any time.  "Γιατί οι πυρήνες προσοχής ...":
//    small tiles of Q and K are brought on chip, the softmax is taken tile by tile
//    and only the running maximum and sum of every query row are kept.
//    "Τι νέο υπάρχει στο FlashAttention 4": the workgroups each own an output tile
//    and stream the matching K/V tiles through on-chip memory.  "Έξυπνος
//    επανακανονισμός Softmax ...": the accumulator is rescaled only when a row's
//    new maximum exceeds the one in use by a significant margin (here: tau, in
//    log2 units).
//  * "PyTorchs FlexAttention mit FlashAttention-4 ist ein Game-Changer" (liora.io),
//    opening section: ALiBi, sliding window, document masking, soft-capping;
//    "Aktuelle Einschränkungen": fully masked blocks are skipped (block sparsity).
//  * "FlashAttention-3: Rekordverdächtige Geschwindigkeit und Präzision bei
//    AI-Modellen" (ctol-digital.de), "Analyse": FP8 inputs with block quantisation.
//
// How it maps onto gfx950 (an MI355X design, not the pages' Hopper/Blackwell one):
//  * one workgroup = 4 waves = 128 query rows of one (b, h); each wave owns 32
//    rows.  The workgroup walks the non-empty 128-key blocks of its row block
//    (from the block map) in 64-key steps.
//  * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (fp8: v_mfma_scale_f32_32x32x64
//    _f8f6f4 with unit scales): K from LDS is the A operand, the wave's Q tile is
//    the B operand and stays in VGPRs for the whole K loop.  In the 32x32 C layout
//    each lane then holds ONE query row (column lane%32) and 16 keys per 32-key
//    block, so the row maximum and row sums are in-lane, finished by one exchange
//    with lane^32.
//  * O^T = V^T . P^T on the same bf16 MFMA.  The contraction index of an MFMA may
//    be permuted freely as long as A and B agree, so the S accumulator registers
//    ARE the B operand of the PV product after a bf16 conversion -- no shuffles.
//    V is staged into LDS transposed in the matching permuted key order, so every
//    A-operand fetch is one 16-byte LDS read.
//  * online softmax in log2 units: x = s * scale * log2(e) (+ modifiers),
//    p = exp2(x - m) on v_exp_f32.  The offset m is replaced (and the O
//    accumulator rescaled) only when a row's maximum exceeds it by more than tau,
//    so p <= 2^tau.  l = sum p (fp32, for LSE); lq = sum of p *as rounded* for the
//    PV MFMA (v_dot2_f32_bf16 against ones), the normaliser of O.
//  * K/V of step j+1 are fetched from HBM into VGPRs while step j computes, then
//    written to the other half of a double-buffered LDS tile: one barrier a step.
//  * LDS rows are XOR-swizzled in 16-byte chunks so MFMA operand reads are free
//    of bank conflicts.
//  * workgroup -> tile mapping is XCD-aware: consecutive workgroups of one XCD
//    (dispatch is round-robin over the 8 XCDs) get consecutive row blocks of the
//    same (b, h), so that head's K/V stays in that XCD's L2; within a head the
//    row blocks run last-first (longest first under a causal mask).
#pragma once

#include <type_traits>

#include "common.hpp"
#include "fwd_args.hpp"

namespace attn119 {


// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // A and B as OCP E4M3 (format 0), unit block scales (E8M0 127 = 2^0).
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ bf16x2 cvt_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_convertvector(v, bf16x2);  // v_cvt_pk_bf16_f32, round to nearest even
}

__device__ __forceinline__ uint32_t as_u32(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ f16x2 cvt_f16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_convertvector(v, f16x2);  // v_cvt_pk_f16_f32, round to nearest even
}

__device__ __forceinline__ f32x16 mfma_f16(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Position of key kk (0..63 within a step) in the permuted order used for the
// transposed V tile: within each 16-key group, bits [b3 b2 b1 b0] -> [b2 b3 b1 b0].
// Lane half hh of the PV MFMA then finds its 8 keys {4hh..4hh+3, 8+4hh..8+4hh+3}
// contiguous, which is exactly the key set its S-accumulator registers hold.
__device__ __forceinline__ int vperm_key(int kk) {
  return (kk & ~15) | ((kk & 4) << 1) | ((kk & 8) >> 1) | (kk & 3);
}

// OCP e4m3 -> bf16 is exact (3 mantissa bits, exponents well inside bf16's range):
// one v_cvt_scalef32_pk_bf16_fp8 (unit scale) per two codes.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 w) {
  return u32x4{as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false)),
               as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true)),
               as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false)),
               as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true))};
}

// e4m3 -> fp16 is exact as well (every e4m3 value, subnormals included, lies inside
// fp16's normal range): v_cvt_scalef32_pk_f16_fp8, unit scale.
__device__ __forceinline__ u32x4 e4m3x8_to_f16x8(u32x2 w) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, true))};
}

// Input modes of the kernel.
//   kInBf16  : bf16 Q/K/V, bf16 MFMA for both products.
//   kInFp8   : e4m3 Q/K/V with block scales; the codes are widened exactly while they
//              are staged (Q, K to bf16; V to fp16) and both products run on 16-bit MFMA
//              with fp32 accumulation: Q.K^T on bf16, P.V on fp16, with P rounded to fp16
//              (8x finer than bf16; P <= 2^tau stays far inside fp16's range).  This is
//              the accurate fp8 mode: gfx950's fp8 MFMA sums its products with a
//              precision of about 2^-13 of the largest one, which inputs with outlier
//              channels turn into score errors of 1e-2.
//   kInFp8Qk8: e4m3 inputs, Q.K^T on the e4m3 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4,
//              twice the bf16 rate, the limited accumulation precision above), PV as kInFp8.
constexpr int kInBf16 = 0, kInFp8 = 1, kInFp8Qk8 = 2;

template <typename T>
__device__ __forceinline__ T ld_global(const void* p) { return *(const T*)p; }

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
//   D       head dim (64 or 128)
//   IN      input mode (kInBf16, kInFp8, kInFp8Qk8)
//   MASKED  positional mask through the block map (else: all keys visible)
//   ALIBI, SOFTCAP  score modifiers
template <int D, int IN, bool MASKED, bool ALIBI, bool SOFTCAP>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(const FwdArgs a) {
  constexpr bool FP8 = IN != kInBf16;          // e4m3 inputs with block scales
  constexpr bool QK8 = IN == kInFp8Qk8;        // Q.K^T on the fp8 MFMA
  constexpr bool WIDEN_K = IN == kInFp8;       // K staged as bf16 from e4m3 codes
  constexpr int BN = 64;                       // keys per step
  constexpr int KRB = D * (FP8 ? 1 : 2);       // bytes per Q/K/V row in HBM
  constexpr int KLB = D * (QK8 ? 1 : 2);       // bytes per K row in LDS
  constexpr int KCPR = KLB / 16;               // 16-byte chunks per LDS K row
  constexpr int KRP = 256 / KLB;               // K rows per 256-byte LDS line
  constexpr int KPASS = (BN * KCPR) / 256;     // K chunks per thread per step
  constexpr int VKPT = D / 32;                 // keys per thread in the V staging
  constexpr int VCPR = D / 8;                  // 8-element d-chunks per V row
  constexpr int NDB = D / 32;                  // 32-wide d blocks of O^T
  constexpr int KT_BYTES = BN * KLB;           // one K tile
  constexpr int VT_BYTES = D * BN * 2;         // one transposed 16-bit V tile (fp16 for fp8)
  constexpr bool LINEAR = !ALIBI && !SOFTCAP;  // score = raw * c

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * KT_BYTES + 2 * VT_BYTES];
  unsigned char* const ks_base = smem;
  unsigned char* const vs_base = smem + 2 * KT_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int N = a.N;
  const int nqb = a.nqb;

  // ---- XCD-aware work mapping (head-major or heaviest-first, chosen on the host) ---
  int bh, qb;
  work_item(a, blockIdx.x, bh, qb);
  const int b = bh / a.H;
  const int h = bh - b * a.H;

  const int q0 = qb * 128;
  const int qrow = q0 + wave * 32 + l32;
  const bool qvalid = qrow < N;
  const size_t head_row0 = (size_t)bh * N;  // Q, O, LSE rows of this head
  const int bkv = kv_head(a, bh);           // its key/value head
  const size_t kv_row0 = (size_t)bkv * N;

  // ---- block-map lookups --------------------------------------------------------
  int nfull, npart;
  const int* flist = nullptr;
  const int* plist = nullptr;
  int lo_q = 0, hi_q = qvalid ? N - 1 : -1;
  bool invalid = false;
  if constexpr (MASKED) {
    const MapHeader* hd = (const MapHeader*)a.map;
    invalid = hd->magic != kMapMagic || hd->B != a.B || hd->N != N || hd->flags != a.mflags ||
              hd->window != a.window;
    const int* cnt = (const int*)(a.map + a.lay.counts) + ((size_t)b * nqb + qb) * 2;
    nfull = min(max(cnt[0], 0), nqb);
    npart = min(max(cnt[1], 0), nqb - nfull);
    flist = (const int*)(a.map + a.lay.idx) + ((size_t)b * nqb + qb) * 2 * nqb;
    plist = flist + nqb;
    if (qvalid) {
      lo_q = ((const int*)(a.map + a.lay.row_lo))[(size_t)b * N + qrow];
      hi_q = ((const int*)(a.map + a.lay.row_hi))[(size_t)b * N + qrow];
    }
    if (a.mflags & kDocument) {
      const int* st = (const int*)(a.map + a.lay.status) + (size_t)b * nqb;
      int bad = 0;
      for (int i = tid; i < nqb; i += 256) bad |= st[i];
      invalid |= __syncthreads_or(bad) != 0;
    }
    if (invalid) { nfull = 0; npart = 0; }
  } else {
    const bool tail = (N & 127) != 0;
    nfull = tail ? nqb - 1 : nqb;
    npart = tail ? 1 : 0;
  }
  const int nsteps = 2 * (nfull + npart);

  // ---- Q tile -> VGPRs (B operand of S^T = K Q^T) ----------------------------------
  constexpr int NQC = QK8 ? D / 64 : D / 16;
  typedef typename std::conditional<QK8, i32x8, bf16x8>::type QFrag;
  QFrag qf[NQC];
  {
    const unsigned char* qp = (const unsigned char*)a.q + (head_row0 + (qvalid ? qrow : 0)) * KRB;
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
      if constexpr (QK8) {
        const u32x4 lo = ld_global<u32x4>(qp + c * 64 + hh * 32);
        const u32x4 hi = ld_global<u32x4>(qp + c * 64 + hh * 32 + 16);
        i32x8 v;
        v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
        v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
        qf[c] = qvalid ? v : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      } else if constexpr (FP8) {
        const u32x4 w = e4m3x8_to_bf16x8(ld_global<u32x2>(qp + c * 16 + hh * 8));
        qf[c] = qvalid ? __builtin_bit_cast(bf16x8, w) : bf16x8{};
      } else {
        const bf16x8 v = ld_global<bf16x8>(qp + (c * 16 + hh * 8) * 2);
        qf[c] = qvalid ? v : bf16x8{};
      }
    }
  }

  // ---- per-row constants --------------------------------------------------------
  float slope2 = 0.f;  // ALiBi slope in log2 units
  if constexpr (ALIBI) {
    const float s = a.alibi_slopes ? a.alibi_slopes[h] : fast_exp2(a.alibi_exp * (float)(h + 1));
    slope2 = s * 1.4426950408889634f;
  }
  const bool alibi_abs = !(a.mflags & kCausal);  // bidirectional masks: -slope*|q-k|
  float sq = 1.f;
  // fp8: P is formed in units of vs/vs_max (the V block scale over the largest V block
  // scale of this head), so that it stays <= 2^tau inside fp16's range whatever the
  // scales are; O is multiplied back by vs_max in the epilogue.
  float vs_max = 1.f;
  if constexpr (FP8) {
    sq = a.q_scale[(size_t)bh * nqb + qb];
    const float* vsr = a.v_scale + (size_t)bkv * nqb;
    float mx = 0.f;
    for (int i = lane; i < nqb; i += 64) mx = __builtin_fmaxf(mx, vsr[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
    vs_max = mx > 0.f ? mx : 1.f;
  }

  // ---- step enumeration -----------------------------------------------------------
  auto step_kb = [&](int s, bool& partial) -> int {
    const int blk = s >> 1;
    partial = blk >= nfull;
    if constexpr (MASKED) {
      const int kb = partial ? plist[blk - nfull] : flist[blk];
      return min(max(kb, 0), nqb - 1);  // a corrupted map never reads out of bounds
    } else {
      return blk;
    }
  };

  // ---- K/V staging: HBM -> VGPRs -> LDS ---------------------------------------------
  const unsigned char* kg = (const unsigned char*)a.k + kv_row0 * KRB;
  const unsigned char* vg = (const unsigned char*)a.v + kv_row0 * KRB;
  typedef typename std::conditional<WIDEN_K, u32x2, u32x4>::type KRow;
  KRow kreg[KPASS];
  typedef typename std::conditional<FP8, u32x2, u32x4>::type VRow;
  VRow vreg[VKPT];
  const int vm = tid / VCPR;   // key group of this thread (VKPT keys)
  const int vc = tid % VCPR;   // d chunk of this thread (8 elements)

  auto load_step = [&](int s) {
    bool partial;
    const int kb = step_kb(s, partial);
    const int k0 = kb * 128 + (s & 1) * BN;
#pragma unroll
    for (int r = 0; r < KPASS; ++r) {
      const int kl = r * (256 / KCPR) + tid / KCPR;
      const int key = k0 + kl;
      const int ch = tid % KCPR;
      if constexpr (WIDEN_K)  // LDS chunk ch holds elements 8ch..8ch+7 = 8 codes
        kreg[r] = key < N ? ld_global<u32x2>(kg + (size_t)key * KRB + ch * 8) : u32x2{0, 0};
      else
        kreg[r] = key < N ? ld_global<u32x4>(kg + (size_t)key * KRB + ch * 16) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < VKPT; ++r) {
      const int key = k0 + vm * VKPT + r;
      if constexpr (FP8)
        vreg[r] = key < N ? ld_global<u32x2>(vg + (size_t)key * KRB + vc * 8) : u32x2{0, 0};
      else
        vreg[r] = key < N ? ld_global<u32x4>(vg + (size_t)key * KRB + vc * 16) : u32x4{0, 0, 0, 0};
    }
  };

  auto store_step = [&](int buf) {
    unsigned char* kbuf = ks_base + buf * KT_BYTES;
#pragma unroll
    for (int r = 0; r < KPASS; ++r) {
      const int kl = r * (256 / KCPR) + tid / KCPR;
      const int ch = tid % KCPR;
      const int phys = ch ^ ((kl / KRP) % KCPR);
      if constexpr (WIDEN_K)
        *(u32x4*)(kbuf + kl * KLB + phys * 16) = e4m3x8_to_bf16x8(kreg[r]);
      else
        *(u32x4*)(kbuf + kl * KLB + phys * 16) = kreg[r];
    }
    // V: VKPT keys x 8 d-values -> transposed pieces of VKPT keys for each d.
    unsigned char* vbuf = vs_base + buf * VT_BYTES;
    uint32_t w[VKPT][4];  // bf16 pairs (d 2j, 2j+1) of each key
#pragma unroll
    for (int r = 0; r < VKPT; ++r) {
      if constexpr (FP8) {
        const u32x4 x = e4m3x8_to_f16x8(vreg[r]);
        w[r][0] = x.x; w[r][1] = x.y; w[r][2] = x.z; w[r][3] = x.w;
      } else {
        w[r][0] = vreg[r].x; w[r][1] = vreg[r].y; w[r][2] = vreg[r].z; w[r][3] = vreg[r].w;
      }
    }
    const int kp = vperm_key(vm * VKPT);  // permuted position of the first key
    const int vchunk = kp >> 3;            // 16-byte chunk within the 128-byte d-row
    const int vwithin = (kp & 7) * 2;      // byte offset inside that chunk
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int d = vc * 8 + dd;
      const int phys = vchunk ^ (((d >> 1) ^ (d >> 4)) & 7);
      unsigned char* dst = vbuf + d * 128 + phys * 16 + vwithin;
      const int j = dd >> 1;
      if constexpr (VKPT == 4) {
        u32x2 piece;
        if (dd & 1) {
          piece.x = (w[0][j] >> 16) | (w[1][j] & 0xffff0000u);
          piece.y = (w[2][j] >> 16) | (w[3][j] & 0xffff0000u);
        } else {
          piece.x = (w[0][j] & 0xffffu) | (w[1][j] << 16);
          piece.y = (w[2][j] & 0xffffu) | (w[3][j] << 16);
        }
        *(u32x2*)dst = piece;
      } else {
        const uint32_t piece = (dd & 1) ? ((w[0][j] >> 16) | (w[1][j] & 0xffff0000u))
                                        : ((w[0][j] & 0xffffu) | (w[1][j] << 16));
        *(uint32_t*)dst = piece;
      }
    }
  };

  // ---- accumulators and softmax state ---------------------------------------------
  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_used = -__builtin_inff();
  float l_sum = 0.f;   // sum of p (unrounded), for LSE
  float lq_sum = 0.f;  // sum of p as rounded for the PV product, the normaliser of O

  if (nsteps > 0) {
    load_step(0);
    store_step(0);
  }
  __syncthreads();

  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  const f16x2 ones_h = {(f16)1.0f, (f16)1.0f};
  typedef typename std::conditional<FP8, f16x8, bf16x8>::type PVFrag;  // P and V^T fragments

  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    bool partial;
    const int kb = step_kb(s, partial);
    const int k0 = kb * 128 + (s & 1) * BN;
    if (s + 1 < nsteps) load_step(s + 1);

    // ---- S^T = K Q^T : two 32-key blocks -------------------------------------------
    const unsigned char* kbuf = ks_base + buf * KT_BYTES;
    f32x16 sacc[2];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      sacc[bk] = f32x16{};
      const int kl = bk * 32 + l32;
      const unsigned char* krow = kbuf + kl * KLB;
      const int swz = (kl / KRP) % KCPR;
#pragma unroll
      for (int c = 0; c < NQC; ++c) {
        if constexpr (QK8) {
          const int c0 = c * 4 + hh * 2;
          const u32x4 lo = *(const u32x4*)(krow + ((c0 ^ swz) * 16));
          const u32x4 hi = *(const u32x4*)(krow + (((c0 + 1) ^ swz) * 16));
          i32x8 kfr;
          kfr[0] = lo.x; kfr[1] = lo.y; kfr[2] = lo.z; kfr[3] = lo.w;
          kfr[4] = hi.x; kfr[5] = hi.y; kfr[6] = hi.z; kfr[7] = hi.w;
          sacc[bk] = mfma_fp8(kfr, qf[c], sacc[bk]);
        } else {
          const bf16x8 kfr = *(const bf16x8*)(krow + (((c * 2 + hh) ^ swz) * 16));
          sacc[bk] = mfma_bf16(kfr, qf[c], sacc[bk]);
        }
      }
    }

    // ---- score modifiers, mask, row maximum ------------------------------------------
    float ct = a.c, sc2t = a.sc2, vs = 1.f, inv_vs = 1.f, log2_vs = 0.f;
    if constexpr (FP8) {
      const float sk = a.k_scale[(size_t)bkv * nqb + kb];
      ct *= sq * sk;
      sc2t *= sq * sk;
      vs = a.v_scale[(size_t)bkv * nqb + kb] / vs_max;
      inv_vs = 1.f / vs;
      log2_vs = log2f(vs);
    }
    // key of register r of block bk: k0 + 32*bk + 8*(r>>2) + 4*hh + (r&3)
    const int kq = k0 + 4 * hh - qrow;  // (key - q) of register 0 of block 0
    if constexpr (!LINEAR) {
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float sraw = sacc[bk][r];
          float x;
          if constexpr (SOFTCAP) {
            const float t = fast_exp2(sraw * sc2t);
            x = __builtin_fmaf(-2.f * a.cap2, fast_rcp(t + 1.f), a.cap2);
          } else {
            x = sraw * ct;
          }
          if constexpr (ALIBI) {
            const float dist = (float)(kq + 32 * bk + 8 * (r >> 2) + (r & 3));
            x = __builtin_fmaf(slope2, alibi_abs ? -__builtin_fabsf(dist) : dist, x);
          }
          sacc[bk][r] = x;
        }
    }
    if (partial) {
      const int rlo = lo_q - (k0 + 4 * hh), rhi = hi_q - (k0 + 4 * hh);
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * bk + 8 * (r >> 2) + (r & 3);
          if (off < rlo || off > rhi) sacc[bk][r] = -__builtin_inff();
        }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = __builtin_fmaxf(mx, sacc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sacc[1][r]);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    if constexpr (LINEAR) mx *= ct;  // ct > 0 keeps the order; -inf stays -inf

    // ---- threshold rescale ----------------------------------------------------------
    const float m_new = __builtin_fmaxf(m_used, mx);
    const bool need = m_new > m_used + a.tau;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? fast_exp2(m_used - m_new) : 1.f;
      m_used = need ? m_new : m_used;
      l_sum *= alpha;
      lq_sum *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
    }
    // exponent offset; -inf only while every key seen so far is hidden (then p = 0)
    const float moff = (m_used == -__builtin_inff() ? 0.f : m_used) - log2_vs;

    // ---- P = exp2(x - m), sums, 16-bit packing ---------------------------------------
    PVFrag pf[4];
    float ls = 0.f, lqs = 0.f;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint32_t pk[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = g * 8 + 2 * t;
          float p0, p1;
          if constexpr (LINEAR) {
            p0 = fast_exp2(__builtin_fmaf(sacc[bk][r], ct, -moff));
            p1 = fast_exp2(__builtin_fmaf(sacc[bk][r + 1], ct, -moff));
          } else {
            p0 = fast_exp2(sacc[bk][r] - moff);
            p1 = fast_exp2(sacc[bk][r + 1] - moff);
          }
          ls += p0 + p1;
          if constexpr (FP8) {
            const f16x2 pb = cvt_f16x2(p0, p1);
            lqs = __builtin_amdgcn_fdot2(pb, ones_h, lqs, false);
            pk[t] = as_u32(pb);
          } else {
            const bf16x2 pb = cvt_bf16x2(p0, p1);
            lqs = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, lqs, false);
            pk[t] = as_u32(pb);
          }
        }
        u32x4 v4 = {pk[0], pk[1], pk[2], pk[3]};
        pf[bk * 2 + g] = __builtin_bit_cast(PVFrag, v4);
      }
    l_sum += ls * inv_vs;
    lq_sum += lqs * inv_vs;

    // ---- O^T += V^T P^T -----------------------------------------------------------
    const unsigned char* vbuf = vs_base + buf * VT_BYTES;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * 32 + l32;
        const int phys = (ks * 2 + hh) ^ (((d >> 1) ^ (d >> 4)) & 7);
        const PVFrag vfr = *(const PVFrag*)(vbuf + d * 128 + phys * 16);
        if constexpr (FP8)
          oacc[db] = mfma_f16(vfr, pf[ks], oacc[db]);
        else
          oacc[db] = mfma_bf16(vfr, pf[ks], oacc[db]);
      }

    if (s + 1 < nsteps) store_step(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------------------
  l_sum += __shfl_xor(l_sum, 32);
  lq_sum += __shfl_xor(lq_sum, 32);
  if (!qvalid) return;
  const float nanv = __builtin_bit_cast(float, 0x7fc00000u);  // quiet NaN (a bit pattern, not folded)
  const float inv = invalid ? nanv : (lq_sum > 0.f ? vs_max / lq_sum : 0.f);
  bf16* op = (bf16*)a.o + (head_row0 + qrow) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 v01 = cvt_bf16x2(oacc[db][4 * i + 0] * inv, oacc[db][4 * i + 1] * inv);
      const bf16x2 v23 = cvt_bf16x2(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
      u32x2 st = {as_u32(v01), as_u32(v23)};
      *(u32x2*)(op + db * 32 + 8 * i + 4 * hh) = st;
    }
  if (hh == 0) {
    float lse;
    if (invalid) lse = nanv;
    else if (l_sum > 0.f) lse = (m_used + log2f(l_sum)) * 0.6931471805599453f;
    else lse = -__builtin_inff();
    a.lse[head_row0 + qrow] = lse;
  }
}

// One launch family per (head dim, input type): the score-modifier and mask
// variants are separate compiled kernels selected here.
template <int D, int IN>
hipError_t launch_fwd_family(const FwdArgs& a, bool masked, bool alibi, bool softcap, hipStream_t st) {
  const dim3 grid((unsigned)(a.B * a.H * a.nqb)), block(256);
#define ATTN119_LAUNCH(M, AL, SC)                                                        \
  if (masked == M && alibi == AL && softcap == SC) {                                     \
    hipLaunchKernelGGL((attn_fwd_kernel<D, IN, M, AL, SC>), grid, block, 0, st, a);      \
    return hipGetLastError();                                                            \
  }
  ATTN119_LAUNCH(false, false, false)
  ATTN119_LAUNCH(false, false, true)
  ATTN119_LAUNCH(false, true, false)
  ATTN119_LAUNCH(false, true, true)
  ATTN119_LAUNCH(true, false, false)
  ATTN119_LAUNCH(true, false, true)
  ATTN119_LAUNCH(true, true, false)
  ATTN119_LAUNCH(true, true, true)
#undef ATTN119_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace attn119

