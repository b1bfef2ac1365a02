// Fused exact-attention forward pass for bf16 inputs on gfx950 (MI355X): the
// software-pipelined kernel.
//
// What is computed (pages, by title and section):
//  * "FlashAttention 4: Γρηγορότερη και Αποδοτική σε Μνήμη Προσοχή για LLMs"
//    (el.linux-konsole.com), "Εισαγωγή" and "Γιατί οι πυρήνες προσοχής ...":
//    scores Q.K^T, softmax, times V, taken tile by tile on chip, keeping only the
//    running maximum and sum of every query row.  "Τι νέο υπάρχει στο FlashAttention
//    4": each workgroup owns an output tile and streams K/V tiles through on-chip
//    memory; the asynchronous pipeline keeps the matrix units busy while the
//    softmax of the previous tile runs.  "Έξυπνος επανακανονισμός Softmax ...": the
//    accumulator is rescaled only when a row's maximum grows past the one in use by
//    a significant margin (tau, in log2 units).
//  * "PyTorchs FlexAttention mit FlashAttention-4 ist ein Game-Changer" (liora.io),
//    opening section: ALiBi, sliding window, document masking, soft-capping;
//    "Aktuelle Einschränkungen": fully masked blocks are skipped (block sparsity).
//
// gfx950 mapping:
//  * a workgroup of 4 waves owns 128 query rows of one (b, h), a wave 32 rows; the
//    non-empty 128-key blocks of the row block are walked in 64-key steps, FULL
//    blocks first (no mask code at all), then PARTIAL ones.
//  * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS as A, the wave's Q tile
//    resident in VGPRs as B): each lane holds one query row and 16 keys per 32-key
//    block, so row maxima and sums are in-lane plus one v_permlane32_swap.
//  * O^T += V^T . P^T on the same MFMA, with the S accumulators (converted to bf16)
//    as the B operand.  V stays row-major in LDS; the V^T A operand is gathered
//    with two ds_read_b64_tr_b16 per MFMA (a 16-lane transposing read), in the key
//    order the S accumulator layout dictates.
//  * K and V tiles move HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//    staging).  The buffer range check returns zeros past the head's last row.
//  * software pipeline, one barrier per step: at step s the workgroup has K(s+1) and
//    V(s) in LDS; it issues the loads of K(s+2) and V(s+1), then the MFMAs of
//    S(s+1) = K(s+1) Q^T interleaved with the exponentials of step s, then
//    O += V(s) P(s) followed by the mask, score modifiers and maximum of S(s+1).
//  * LDS layouts are XOR-swizzled in 16-byte chunks so that both the K reads
//    (ds_read_b128) and the V transposing reads are free of bank conflicts.
//  * score modifiers are arranged to cost little per element:
//      LINEAR   x = s*c                       max on raw s, p = exp2(s*c - m)
//      SOFTCAP  x = cap*tanh(s*scale/cap)     monotone in s: max on raw s; in the
//               (log2 units)                  P.V phase r = 1/(exp2(2 s c/cap)+1),
//                                             then p = exp2(cap' - m - 2 cap' r)
//      ALIBI_C  x = s*c + slope*(k - q)       causal masks: y = s*c + slope*(k - k0
//                                             - 4hh) per element; the per-row part
//                                             slope*(k0 + 4hh - q) moves into m
//      GENERIC  anything else (ALiBi with softcap or a bidirectional mask)
#pragma once

#include <type_traits>
#include <utility>

#include "common.hpp"
#include "fwd_args.hpp"

namespace attn119 {
namespace bf16path {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// score-modifier modes
constexpr int kLinear = 0, kSoftcap = 1, kAlibiCausal = 2, kGeneric = 3;
// P.V precision (PV): the 16-bit MFMA; e4m3 P; E2M1 P with E8M0 block scales
constexpr int kPv16 = 0, kPvE4m3 = 1, kPvFp4 = 2;

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ bf16x2 to_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_convertvector(v, bf16x2);  // v_cvt_pk_bf16_f32, round to nearest even
}

// Pins v to this point of the program (an empty volatile asm that reads and rewrites
// it in a VGPR): whatever computes v stays before it, whatever uses the new v stays
// after it, so neither can drift across the scheduling fences around it.
template <typename T>
__device__ __forceinline__ void pin(T& v) {
  static_assert(sizeof(T) == 4, "one VGPR");
  asm volatile("" : "+v"(v));
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One 16-byte chunk per lane from a buffer into LDS at lds_base + 16*lane, untracked by
// the compiler (every step waits for its tiles itself, in wait_tiles, before its barrier).
__device__ __forceinline__ void load_lds16(u32x4 rsrc, lds_u8* lds_base, int voffset) {
  dma_to_lds<16>(rsrc, lds_base, voffset);
}

// e4m3 (OCP) codes widen exactly to bf16 and to fp16 (3 mantissa bits; every e4m3
// exponent, subnormals included, lies inside both formats' normal range): one
// v_cvt_scalef32_pk_*_fp8 with unit scale per two codes.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
}
__device__ __forceinline__ u32x4 e4m3x8_to_f16x8(uint32_t lo, uint32_t hi) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true))};
}

// key offset (within a 64-key step, minus 4*hh) of accumulator register r of block bk
__host__ __device__ constexpr int key_off(int bk, int r) { return 32 * bk + 8 * (r >> 2) + (r & 3); }

//   D       head dim (64 or 128)
//   FP8     e4m3 Q/K/V codes with per-(b, h, 128-row block) fp32 scales: the codes are
//           widened exactly as they are staged (Q, K to bf16, V to fp16); Q.K^T runs on
//           the bf16 MFMA, P.V on the fp16 MFMA with P rounded to fp16, in units of
//           vs_kb / vs_max (the key block's V scale over the head's largest), so that
//           P <= 2^tau stays inside fp16 whatever the scales; O is multiplied back by
//           vs_max and normalised by the fp32 row sum (fp16 P is within 2^-11 of it).
//   QK8     (with FP8) Q.K^T on the e4m3 MFMA instead: K codes go to LDS as they are (direct
//           loads), Q codes stay in VGPRs, S = K.Q^T on v_mfma_scale_f32_32x32x64_f8f6f4
//           (unit block scales; the fp32 scales are applied to S as above).  The MFMA
//           sums a 64-term dot product with about 14 bits below its largest product
//           (measured; truncating), so a score dominated by a few large products carries
//           an error of that size.
//   COUNT   also count each row's rescale events into a.rescale_counts (a separate
//           instantiation, so that the counter costs the other kernels no register)
//   PV      P.V precision: 0 the 16-bit MFMA above; with QK8 (no positional mask, linear
//           scores, D = 128) also P on the f8f6f4 MFMA with the V codes as they are:
//           kPvE4m3, P rounded to e4m3; kPvFp4, P rounded to E2M1 with one E8M0 scale
//           per lane's 32 keys (the smallest power of two that holds their largest value,
//           "Direct-P" from the exponentials); O is normalised by the sum of the rounded P
//   MASKED  positional mask through the block map (else: all keys visible)
//   MODE    score-modifier mode (kLinear, kSoftcap, kAlibiCausal, kGeneric)
//   GALIBI, GSOFTCAP  modifiers of the generic mode
template <int D, bool FP8, bool QK8, bool COUNT, int PV, bool MASKED, int MODE, bool GALIBI, bool GSOFTCAP>
__global__ void __launch_bounds__(256, 2) attn_fwd_bf16_kernel(const FwdArgs a) {
  static_assert(PV == 0 || (QK8 && !MASKED && MODE == kLinear && D == 128 && !COUNT),
                "the fp8/fp4 P.V runs with the e4m3 Q.K^T, no positional mask, linear scores, d = 128");
  static_assert(FP8 || !QK8, "the e4m3 Q.K^T takes e4m3 inputs");
  static_assert(!(QK8 && MODE == kSoftcap), "softcap with e4m3 Q.K^T runs in the generic mode");
  constexpr int BN = 64;                 // keys per step
  constexpr int ROWB = D * 2;            // bytes per 16-bit row of Q/K/V (LDS; HBM for bf16)
  constexpr int HROWB = FP8 ? D : D * 2;  // bytes per row in HBM
  constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
  constexpr int RP256 = 256 / ROWB;      // rows per 256-byte LDS line
  constexpr int TILE = BN * ROWB;        // bytes of one K or V tile
  constexpr int LOADS = TILE / 1024;     // 1 KiB direct loads per tile
  constexpr int LPW = LOADS / 4;         // ... per wave
  constexpr int RPL = 1024 / ROWB;       // rows per direct load
  // K in LDS: 16-bit rows, or e4m3 codes with QK8
  constexpr int KROWB = QK8 ? D : ROWB;  // bytes per K row in LDS
  constexpr int KCPR = KROWB / 16;
  constexpr int KRP256 = 256 / KROWB;
  constexpr int KLPW = BN * KROWB / 1024 / 4;  // 1 KiB direct K loads per wave
  constexpr int KRPL = 1024 / KROWB;
  constexpr bool DIRECT_K = !FP8 || QK8;  // K tiles by direct HBM -> LDS loads
  constexpr bool DIRECT_V = !FP8 || PV != 0;  // V tiles likewise (else staged and widened)
  // V in LDS: 16-bit rows, or e4m3 codes for the fp8/fp4 P.V
  constexpr int VROWB = PV ? D : ROWB;
  constexpr int VCPR = VROWB / 16;
  constexpr int VLPW = BN * VROWB / 1024 / 4;
  constexpr int VRPL = 1024 / VROWB;
  constexpr int NQC = QK8 ? D / 64 : D / 16;  // MFMA k steps of S (64- or 16-wide d chunks)
  constexpr int NDB = D / 32;            // 32-wide d blocks of O^T
  typedef typename std::conditional<QK8, i32x8, bf16x8>::type KF;  // K fragment / Q operand

  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases stay scalar
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int N = a.N;
  const int nqb = a.nqb;

  // ---- XCD-aware work mapping (head-major or heaviest-first, chosen on the host) -----
  int bh, qb;
  work_item(a, blockIdx.x, bh, qb);
  const int b = bh / a.H;
  const int h = bh - b * a.H;

  const int q0 = qb * 128;
  const int qrow = q0 + wave * 32 + l32;
  const bool qvalid = qrow < N;
  const size_t head_row0 = (size_t)bh * N;                 // Q, O, LSE rows of this head
  const int bkv = kv_head(a, bh);                          // its key/value head
  const size_t kv_row0 = (size_t)bkv * N;

  // ---- block-map lookups (scalar loads through the constant address space: the map
  //      is read-only here and every index is uniform over the workgroup) -------------
  typedef const __attribute__((address_space(4))) int cint;
  int nfull, npart;
  int lo_q = 0, hi_q = qvalid ? N - 1 : -1;
  int kb_first = 0;  // first block of the order (masked: read beside the counts)
  bool invalid = false;
  // Every mask here makes row q see the keys [lo(q), hi(q)], both ends non-decreasing in
  // q and q itself inside (a document mask within documents whose ids do not decrease --
  // a batch row where they do is poisoned below).  So the block's rows r0..r1 together see
  // [lo(r0), hi(r1)] without a gap: the non-empty key blocks are the range ua..ub; a block
  // is FULL when it lies in every row's interval, [lo(r1), hi(r0)], and the block has 128
  // rows; the PARTIAL ones are the pl blocks left of the FULL range and those right of it
  // -- the block map's lists, in the map's order (PARTIAL ascending, then FULL ascending):
  // entry j is block map_entry(j).  Without a map (causal and window masks) lo and hi
  // follow from the flags; with one they are the map's row intervals, of which the four
  // of rows r0 and r1 give the ranges (the map's lists are not read).
  const bool derive = MASKED && a.map == nullptr;
  int ua = 0, fa = 0, fb = -1, pl = 0;
  auto map_entry = [&](int j) -> int {
    return j < pl ? ua + j : (j < npart ? fb + 1 + (j - pl) : fa + (j - npart));
  };
  auto set_ranges = [&](int lo0, int lo1, int hi0, int hi1, int r0, int r1) {
    ua = min(max(lo0 >> 7, 0), nqb - 1);
    const int ub = min(max(hi1 >> 7, ua), nqb - 1);
    fa = max(ua, (lo1 + 127) >> 7);
    fb = min(ub, ((hi0 + 1) >> 7) - 1);
    if (r1 - r0 != 127 || fa > fb) { fa = ub + 1; fb = ub; }  // no FULL block
    nfull = fb - fa + 1;
    npart = ub - ua + 1 - nfull;
    pl = fa - ua;
    kb_first = map_entry(0);
  };
  if (MASKED && derive) {
    const int W = a.window;
    const uint32_t mf = a.mflags;
    auto lo_of = [&](int q) { return (mf & kWindow) ? max(0, q - (W - 1)) : 0; };
    auto hi_of = [&](int q) {
      return (mf & kCausal) ? q : ((mf & kWindow) ? min(N - 1, q + (W - 1)) : N - 1);
    };
    const int r0 = q0, r1 = min(N, q0 + 128) - 1;
    set_ranges(lo_of(r0), lo_of(r1), hi_of(r0), hi_of(r1), r0, r1);
    if (qvalid) {
      lo_q = lo_of(qrow);
      hi_q = hi_of(qrow);
    }
  } else if constexpr (MASKED) {
    const __attribute__((address_space(4))) MapHeader* hd =
        (const __attribute__((address_space(4))) MapHeader*)a.map;
    invalid = hd->magic != kMapMagic || hd->B != a.B || hd->N != N || hd->flags != a.mflags ||
              hd->window != a.window || hd->compact != a.compact;
    {
      cint* rlo = (cint*)(a.map + a.lay.row_lo) + (size_t)b * N;
      cint* rhi = (cint*)(a.map + a.lay.row_hi) + (size_t)b * N;
      const int r0 = q0, r1 = min(N, q0 + 128) - 1;
      set_ranges(rlo[r0], rlo[r1], rhi[r0], rhi[r1], r0, r1);
    }
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
  const int nblk = nfull + npart;
  const int nsteps = 2 * nblk;

  // Steps walk the PARTIAL blocks first (masked, one step at a time), then the FULL
  // blocks (software-pipelined, no mask code).  First key of step s:
  // (masked: the block order sits in VGPR lanes -- lane i of kbv[r] holds block
  // 64r + i -- so a lookup is one v_readlane with no memory latency; orders longer
  // than 128 blocks read the rest from the map)
  constexpr int NKV = 2;
  int kbv[NKV];
  if constexpr (MASKED) {
#pragma unroll
    for (int r = 0; r < NKV; ++r) {
      const int j = 64 * r + lane;
      int kb = 0;
      if (j < nblk) kb = map_entry(j);
      kbv[r] = min(max(kb, 0), nqb - 1);  // (never outside the head, whatever the map holds)
    }
  }
  auto step_k0 = [&](int s) -> int {
    const int blk = s >> 1;
    int kb;
    if constexpr (MASKED) {
      if (blk < 64) {
        kb = __builtin_amdgcn_readlane(kbv[0], blk);
      } else if (blk < 64 * NKV) {
        kb = __builtin_amdgcn_readlane(kbv[1], blk - 64);
      } else {
        kb = min(max(map_entry(blk), 0), nqb - 1);
      }
    } else {
      kb = blk < npart ? nqb - 1 : blk - npart;  // the ragged tail block is the PARTIAL one
    }
    return kb * 128 + (s & 1) * BN;
  };
  // the same for the steps of the first block, without reading the block order
  auto step_k0_first = [&](int s) -> int {
    if constexpr (MASKED) return s < 2 ? kb_first * 128 + (s & 1) * BN : step_k0(s);
    else return step_k0(s);
  };

  // ---- Q tile -> VGPRs (B operand of S^T = K Q^T) ----------------------------------------
  KF qf[NQC];
  if constexpr (QK8) {
    // 32 codes per lane: d = 64c + 32hh .. +31 of the lane's row (the f8f6f4 operand layout)
    const unsigned char* qp = (const unsigned char*)a.q + (head_row0 + (qvalid ? qrow : 0)) * D;
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
      const u32x4 lo = *(const u32x4*)(qp + c * 64 + hh * 32);
      const u32x4 hi = *(const u32x4*)(qp + c * 64 + hh * 32 + 16);
      const i32x8 v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      qf[c] = qvalid ? v : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  } else if constexpr (FP8) {
    const unsigned char* qp = (const unsigned char*)a.q + (head_row0 + (qvalid ? qrow : 0)) * D;
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
      const u32x2 w = *(const u32x2*)(qp + c * 16 + hh * 8);
      const bf16x8 v = __builtin_bit_cast(bf16x8, e4m3x8_to_bf16x8(w.x, w.y));
      qf[c] = qvalid ? v : bf16x8{};
    }
  } else {
    const bf16* qp = (const bf16*)a.q + (head_row0 + (qvalid ? qrow : 0)) * D;
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
      const bf16x8 v = *(const bf16x8*)(qp + c * 16 + hh * 8);
      qf[c] = qvalid ? v : bf16x8{};
    }
  }

  // ---- direct HBM -> LDS loads ---------------------------------------------------------
  // K rows: 16-byte chunk ch of row r sits at chunk position ch ^ kswz(r).
  // V rows: chunk ch of row r sits at ch ^ vswz(r).
  auto kswz = [](int r) { return (r / KRP256) % KCPR; };
  // (e4m3 V rows for the fp8/fp4 P.V: chunk ch of row r at ch ^ 2(bit1(r) | bit3(r) << 1),
  // which spreads the 8 rows one transposing read touches over distinct banks)
  auto vswz = [](int r) {
    if constexpr (PV != 0) return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
    else return 4 * ((r / RP256) % (CPR / 4));
  };
  // The buffer descriptor of a step starts at its first key row and covers the rows
  // left in the head, so every row past N reads as zero (range-checked on the lane
  // offset; no address ever leaves the head).
  const unsigned char* const kbase = (const unsigned char*)a.k + kv_row0 * HROWB;
  const unsigned char* const vbase = (const unsigned char*)a.v + kv_row0 * HROWB;
  auto rsrc = [&](const unsigned char* base, int k0) {
    return dma_rsrc(base + (size_t)k0 * HROWB, max(N - k0, 0) * HROWB);
  };
  // (the staged fp8 tiles load into registers through the compiler-tracked builtin)
  auto rsrc_reg = [&](const unsigned char* base, int k0) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)k0 * HROWB), (short)0,
                                             max(N - k0, 0) * HROWB, 0x00020000);
  };
  int koff[KLPW], voff[VLPW];  // byte offsets within a tile, per direct load of this wave
#pragma unroll
  for (int r = 0; r < KLPW; ++r) {
    const int ld = wave * KLPW + r;
    const int row = ld * KRPL + lane / KCPR;
    koff[r] = row * KROWB + ((lane % KCPR) ^ kswz(row)) * 16;
  }
#pragma unroll
  for (int r = 0; r < VLPW; ++r) {
    const int ld = wave * VLPW + r;
    const int row = ld * VRPL + lane / VCPR;
    voff[r] = row * VROWB + ((lane % VCPR) ^ vswz(row)) * 16;
  }
  auto issue_k = [&](int k0, lds_u8* dst) {
    const u32x4 rs = rsrc(kbase, k0);
#pragma unroll
    for (int r = 0; r < KLPW; ++r) load_lds16(rs, dst + (wave * KLPW + r) * 1024, koff[r]);
  };
  auto issue_v = [&](int k0, lds_u8* dst) {
    const u32x4 rs = rsrc(vbase, k0);
#pragma unroll
    for (int r = 0; r < VLPW; ++r) load_lds16(rs, dst + (wave * VLPW + r) * 1024, voff[r]);
  };

  // ---- fp8: staging through VGPRs ------------------------------------------------------
  // Thread t stages SCH 8-code chunks of row t/4 of a 64-row tile: stage_* loads them into
  // registers (range-checked: rows past N read as zero codes), commit_*_chunk widens one
  // (8 codes -> one 16-byte chunk of the 16-bit row) and writes it to the tile in the
  // swizzled layouts above.  A tile is staged one step before it is committed, so the load
  // latency is spent under a whole step.
  // Which chunk a thread commits in slot j is chosen by its LDS position, not its index:
  // LDS serves a 16-byte write to 8 lanes per cycle, so the 8 lanes of a group (2 rows x 4
  // threads) must hit 8 different 16-byte slots of a 128-byte line (and the 16 lanes of 4
  // rows 16 different slots of 256 bytes).  Slot j of thread (row r, q = t%4) writes
  // position p = 4(j ^ (r%4)) + q (d = 128) or 2q + (j ^ r0 ^ r1) (d = 64, r0 r1 the low
  // bits of r); for a fixed row these cover every position once, and the chunk that
  // belongs there, p ^ swizzle(r), is the one the thread loads for slot j.
  constexpr int SCH = D / 32;      // 8-code chunks per thread per tile
  u32x2 kst[FP8 ? SCH : 1], vst[FP8 ? SCH : 1];
  int kldo[FP8 ? SCH : 1], vldo[FP8 ? SCH : 1], stpos[FP8 ? SCH : 1];
  const int srow = tid >> 2;
  if constexpr (FP8) {
    const int q = tid & 3;
#pragma unroll
    for (int j = 0; j < SCH; ++j) {
      const int p = D == 128 ? 4 * (j ^ (srow & 3)) + q : 2 * q + (j ^ (srow & 1) ^ ((srow >> 1) & 1));
      stpos[j] = srow * ROWB + p * 16;
      kldo[j] = srow * D + (p ^ kswz(srow)) * 8;
      vldo[j] = srow * D + (p ^ vswz(srow)) * 8;
    }
  }
  auto stage_k = [&](int k0) {
    if constexpr (!DIRECT_K) {
      const __amdgpu_buffer_rsrc_t rs = rsrc_reg(kbase, k0);
#pragma unroll
      for (int j = 0; j < SCH; ++j)
        kst[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, kldo[j], 0, 0));
    }
  };
  auto stage_v = [&](int k0) {
    if constexpr (FP8) {
      const __amdgpu_buffer_rsrc_t rs = rsrc_reg(vbase, k0);
#pragma unroll
      for (int j = 0; j < SCH; ++j)
        vst[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, vldo[j], 0, 0));
    }
  };
  auto commit_k_chunk = [&](lds_u8* dst, int j) {
    if constexpr (!DIRECT_K)
      *(__attribute__((address_space(3))) u32x4*)(dst + stpos[j]) = e4m3x8_to_bf16x8(kst[j].x, kst[j].y);
  };
  auto commit_v_chunk = [&](lds_u8* dst, int j) {
    if constexpr (FP8)
      *(__attribute__((address_space(3))) u32x4*)(dst + stpos[j]) = e4m3x8_to_f16x8(vst[j].x, vst[j].y);
  };
  auto commit_k = [&](lds_u8* dst) {
#pragma unroll
    for (int j = 0; j < SCH; ++j) commit_k_chunk(dst, j);
  };
  auto commit_v = [&](lds_u8* dst) {
#pragma unroll
    for (int j = 0; j < SCH; ++j) commit_v_chunk(dst, j);
  };
  // the tiles of step s (bf16: requested straight into LDS; fp8: committed from the
  // staging registers, then the tiles of the step after are staged)
  auto wait_tiles = [&]() {
    if constexpr (DIRECT_K && DIRECT_V) wait_vmem();  // this wave's direct loads
    else if constexpr (DIRECT_K) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");  // both kinds
    else asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's chunk writes
  };

  // ---- LDS read addressing -------------------------------------------------------------
  // K (A operand of S^T): lane reads row 32*bk + l32, chunk 2c + hh (16-bit rows), or the
  // two chunks 4c + 2hh and 4c + 2hh + 1 (e4m3 rows: 32 codes per lane).
  int kread[NQC][QK8 ? 2 : 1];
  {
    const int sw = kswz(l32);  // the same for rows l32 and 32 + l32
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
      if constexpr (QK8) {
        kread[c][0] = l32 * KROWB + ((4 * c + 2 * hh) ^ sw) * 16;
        kread[c][1] = l32 * KROWB + ((4 * c + 2 * hh + 1) ^ sw) * 16;
      } else {
        kread[c][0] = l32 * ROWB + ((2 * c + hh) ^ sw) * 16;
      }
    }
  }
  // V^T (A operand of O^T): two 16-lane transposing reads per MFMA.  Within a 16-lane
  // group, source lane 4e + a addresses key row key_e and the 4 d values
  // 32 db + 16 dh + 4a .. +3; the read hands lane 4a + b the value of d = ... + 4a + b
  // for the 4 keys key_0..key_3.  key_e = 16 ks + 8 t + 4 hh + e.
  int vread[NDB];
  {
    const int e = (lane & 15) >> 2, aa = lane & 3, dh = (lane >> 4) & 1;
    const int row = 4 * hh + e;  // + 16 ks + 8 t (multiples of 8 keep vswz unchanged)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int chunk = 4 * db + 2 * dh + (aa >> 1);
      vread[db] = row * ROWB + (chunk ^ vswz(row)) * 16 + (aa & 1) * 8;
    }
  }
  // V^T (A operand of the f8f6f4 P.V, e4m3 codes): 32 keys of one d per lane from four
  // 8-bit transposing reads.  Within a 16-lane group, result lane i, byte e comes from
  // source lane 2e + i/8, byte i % 8 (measured on gfx950): source lane 2e + c addresses
  // key row row_e(r) and the 8 d values 32 db + 16 mh + 8c .. +7, and result lane i holds
  // d = 32 db + 16 mh + i for the 8 keys.  The keys follow the P operand: e4m3 P lane
  // (n, hh) byte j is the score of key 32(j/16) + 8(j%16/4) + j%4 + 4 hh (the S accumulator
  // order), and an e2m1 B lane of half hh pairs its nibble p with A half p/16, byte
  // 16 hh + p%16 (measured), so the A bytes of half hh' are, per read r (bytes 8r..8r+7):
  //   e4m3 P: rows 16 r + 8(e/4) + e%4 + 4 hh'
  //   e2m1 P: rows 32 hh' + 16(r%2) + 8(e/4) + e%4 + 4(r/2)
  int vread8[PV ? NDB : 1];
  if constexpr (PV != 0) {
    const int src = lane & 15, e = src >> 1, c = src & 1, G = lane >> 4, hp = G >> 1, mh = G & 1;
    const int hsw = ((e >> 1) & 1) | (((e >> 2) & 1) << 1);  // the rows' swizzle (bits 1, 3 of the row)
    const int L = PV == kPvE4m3 ? 8 * (e >> 2) + (e & 3) + 4 * hp : 32 * hp + 8 * (e >> 2) + (e & 3);
#pragma unroll
    for (int db = 0; db < NDB; ++db) vread8[db] = L * VROWB + 32 * (db ^ hsw) + 16 * mh + 8 * c;
  }
  auto vfrag8 = [&](const lds_u8* vt, int db) -> i32x8 {
    typedef int v2i __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i lds_v2i;
    v2i w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int roff = PV == kPvE4m3 ? 16 * r : 16 * (r & 1) + 4 * (r >> 1);
      w[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vt + vread8[PV ? db : 0] + roff * VROWB));
    }
    return i32x8{w[0][0], w[0][1], w[1][0], w[1][1], w[2][0], w[2][1], w[3][0], w[3][1]};
  };
  auto kfrag = [&](const lds_u8* kt, int bk, int c) -> KF {
    if constexpr (QK8) {
      typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
      const u32x4 lo = *(const lds_u32x4*)(kt + bk * 32 * KROWB + kread[c][0]);
      const u32x4 hi = *(const lds_u32x4*)(kt + bk * 32 * KROWB + kread[c][1]);
      return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
      return *(const __attribute__((address_space(3))) bf16x8*)(kt + bk * 32 * ROWB + kread[c][0]);
    }
  };
  // S^T += K Q^T for one MFMA k step
  auto qk_mma = [&](const KF& ka, const KF& qb, const f32x16& acc) -> f32x16 {
    if constexpr (QK8)  // A and B as OCP e4m3 (format 0), unit E8M0 block scales (127 = 2^0)
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qb, acc, 0, 0, 0, 127, 0, 127);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb, acc, 0, 0, 0);
  };
  auto vfrag = [&](const lds_u8* vt, int ks, int db) {
    const lds_u8* base = vt + ks * 16 * ROWB + vread[db];
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * ROWB));
    const short __attribute__((ext_vector_type(8))) w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w);
  };

  // ---- per-row constants ------------------------------------------------------------------
  float slope2 = 0.f;  // ALiBi slope in log2 units
  if constexpr (MODE == kAlibiCausal || GALIBI) {
    const float sl = a.alibi_slopes ? a.alibi_slopes[h] : exp2_(a.alibi_exp * (float)(h + 1));
    slope2 = sl * 1.4426950408889634f;
  }
  const bool alibi_abs = !(a.mflags & kCausal);  // bidirectional masks: -slope*|q-k|
  const float cap2 = a.cap2, tau = a.tau;
  // Score multipliers: c = scale*log2e and sc2 = 2c/cap for the exponentials of the
  // current step (ct, sc2) and for the maximum of the step being prepared (ctp, sc2p);
  // for fp8 both carry the Q and K block scales sq*sk, which change with the key block.
  float ct = a.c, sc2 = a.sc2, ctp = a.c, sc2p = a.sc2;
  // fp8: V block scale of the current step over the head's largest (log2 and inverse)
  float lvs = 0.f, ivs = 1.f;
  float sq = 1.f, vs_max = 1.f, lvs_max = 0.f;
  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat* const ksc = FP8 ? (cfloat*)a.k_scale + (size_t)bkv * nqb : nullptr;
  cfloat* const vsc = FP8 ? (cfloat*)a.v_scale + (size_t)bkv * nqb : nullptr;
  if constexpr (FP8) {
    sq = ((cfloat*)a.q_scale)[(size_t)bh * nqb + qb];
    float mx = 0.f;
    for (int i = lane; i < nqb; i += 64) mx = __builtin_fmaxf(mx, a.v_scale[(size_t)bkv * nqb + i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
    vs_max = mx > 0.f ? mx : 1.f;
    lvs_max = __builtin_amdgcn_logf(vs_max);
  }
  // the multipliers of the step whose first key is k0 (for the maximum / the exponentials)
  auto scales_p = [&](int k0) {
    if constexpr (FP8) {
      const float f = sq * ksc[k0 >> 7];
      ctp = a.c * f;
      sc2p = a.sc2 * f;
    }
  };
  auto scales_e = [&](int k0) {
    if constexpr (FP8) {
      const float f = sq * ksc[k0 >> 7];
      ct = a.c * f;
      sc2 = a.sc2 * f;
      // log2(vs_kb / vs_max) and vs_max / vs_kb without divisions (per step, per lane: the
      // hardware reciprocal's 1-ulp error only scales this step's share of the LSE sum)
      const float vk = vsc[k0 >> 7];
      lvs = __builtin_amdgcn_logf(vk) - lvs_max;
      ivs = vs_max * __builtin_amdgcn_rcpf(vk);
    }
  };
  const float ninf = -__builtin_inff();

  // ---- state ----------------------------------------------------------------------------
  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_used = ninf;
  float l_sum = 0.f;   // row sum of p (fp32, before rounding): LSE; for bf16 also the normaliser of O
  int nres = 0;        // steps in which this row's offset was replaced (rescale events)
  float lq_sum = 0.f;  // fp8/fp4 P.V: row sum of P as rounded for the MFMA, the normaliser of O

  // ---- score modifiers, mask and row maximum ---------------------------------------------
  // Score of one accumulator element before the maximum is taken (kq = k0 + 4hh - q):
  // ALiBi-causal and generic modes transform it here; linear and softcap keep raw s
  // (both are monotone in s, so the maximum is taken on s and converted afterwards).
  auto xform = [&](float sraw, int bk, int r, int kq) -> float {
    if constexpr (MODE == kAlibiCausal) {
      // y = s*c + slope*key_off; the row part slope*(k0 + 4hh - q) is added to the max
      // and subtracted from the exponent offset instead
      return __builtin_fmaf(sraw, ctp, slope2 * (float)key_off(bk, r));
    } else if constexpr (MODE == kGeneric) {
      float x;
      if constexpr (GSOFTCAP) x = __builtin_fmaf(-2.f * cap2, rcp_(exp2_(sraw * sc2p) + 1.f), cap2);
      else x = sraw * ctp;
      if constexpr (GALIBI) {
        const float dist = (float)(kq + key_off(bk, r));
        x = __builtin_fmaf(slope2, alibi_abs ? -__builtin_fabsf(dist) : dist, x);
      }
      return x;
    } else {
      return sraw;
    }
  };
  // Row maximum in log2 units (both lane halves) from the in-lane maximum mx of the
  // transformed scores of a step whose first key is k0; -inf for a row with no visible key.
  auto finalize = [&](float mx, int k0) -> float {
    if constexpr (MODE == kAlibiCausal) mx = __builtin_fmaf(slope2, (float)(k0 + 4 * hh - qrow), mx);
    mx = pair_max(mx);
    if constexpr (MODE == kLinear) {
      mx *= ctp;  // ctp > 0 keeps the order; -inf stays -inf
    } else if constexpr (MODE == kSoftcap) {
      const float xm = __builtin_fmaf(-2.f * cap2, rcp_(exp2_(mx * sc2p) + 1.f), cap2);
      mx = mx == ninf ? ninf : xm;
    }
    return mx;
  };
  // Transform, mask (MASK: PARTIAL steps) and row maximum of the S^T accumulators of a
  // step whose first key is k0.  Hidden keys become -inf.  With RAW false a softcap step
  // also leaves r = 1 / (exp2(2 s c / cap) + 1) in sacc (r = +inf for a hidden key, so
  // that p = 0); with RAW true softcap scores stay raw and the exponential phase forms r.
  auto prepare = [&](auto mask_tag, auto raw_tag, f32x16 (&sacc)[2], int k0) -> float {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool RAW = decltype(raw_tag)::value;
    const int kq = k0 + 4 * hh - qrow;
    const int rlo = lo_q - (k0 + 4 * hh), rhi = hi_q - (k0 + 4 * hh);
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[bk][r] = xform(sacc[bk][r], bk, r, kq);
    if constexpr (MASK) {
      // Only the bounds that hide a key of this step in some lane of the wave are
      // applied (wave-uniform branches): a causal diagonal step needs the upper bound
      // alone, a window's far edge the lower alone, and a wave whose 32 x 64 tile is
      // all visible none.  Key offsets run from 0 to key_off(1, 15).
      constexpr int kOffMax = key_off(1, 15);
      const bool need_lo = __builtin_amdgcn_ballot_w64(rlo > 0) != 0;
      const bool need_hi = __builtin_amdgcn_ballot_w64(rhi < kOffMax) != 0;
      if (need_lo && need_hi) {
#pragma unroll
        for (int bk = 0; bk < 2; ++bk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = key_off(bk, r);
            sacc[bk][r] = (off < rlo || off > rhi) ? ninf : sacc[bk][r];
          }
      } else if (need_hi) {
#pragma unroll
        for (int bk = 0; bk < 2; ++bk)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[bk][r] = key_off(bk, r) > rhi ? ninf : sacc[bk][r];
      } else if (need_lo) {
#pragma unroll
        for (int bk = 0; bk < 2; ++bk)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[bk][r] = key_off(bk, r) < rlo ? ninf : sacc[bk][r];
      }
    }
    float mx = ninf;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sacc[bk][r]);
    if constexpr (MODE == kSoftcap && !RAW) {
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float sv = sacc[bk][r];
          const float rr = rcp_(exp2_(sv * sc2p) + 1.f);
          sacc[bk][r] = sv == ninf ? __builtin_inff() : rr;
        }
    }
    return finalize(mx, k0);
  };

  // Exponentials of two scores, in three stages that the pipelined loop issues in
  // different slots (the non-pipelined paths run them back to back):
  //   pre  (softcap scores still raw only): r = 1 / (exp2(2 s c / cap) + 1)
  //   expo p = 2^(score - moff) for the mode's score form
  //   pack the bf16 pair of the B operand; adds both values to the row sum
  auto p_pre = [&](float sv) -> float { return rcp_(exp2_(sv * sc2) + 1.f); };
  auto p_exp = [&](float sv, float moff) -> float {
    if constexpr (MODE == kLinear) return exp2_(__builtin_fmaf(sv, ct, -moff));
    else if constexpr (MODE == kSoftcap) return exp2_(__builtin_fmaf(-2.f * cap2, sv, cap2 - moff));
    else return exp2_(sv - moff);
  };
  auto p_pack = [&](float p0, float p1, float& ls) -> uint32_t {
    ls += p0 + p1;
    if constexpr (FP8) {
      const f32x2 v = {p0, p1};
      const f16x2 pb = __builtin_convertvector(v, f16x2);  // v_cvt_pk_f16_f32, round to nearest even
      return __builtin_bit_cast(uint32_t, pb);
    } else {
      return __builtin_bit_cast(uint32_t, to_bf16x2(p0, p1));
    }
  };
  // all three stages of one pair (RAW: softcap scores untransformed)
  auto ppair = [&](auto raw_tag, float s0, float s1, float moff, float& ls) -> uint32_t {
    constexpr bool RAW = decltype(raw_tag)::value;
    if constexpr (MODE == kSoftcap && RAW) {
      s0 = p_pre(s0);
      s1 = p_pre(s1);
    }
    return p_pack(p_exp(s0, moff), p_exp(s1, moff), ls);
  };
  // P of one 16-key slice (registers 8g..8g+7 of block bk) as the bf16 B operand
  auto pslice = [&](auto raw_tag, const f32x16& sacc, int g, float moff, float& ls) -> bf16x8 {
    uint32_t pk[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) pk[t] = ppair(raw_tag, sacc[g * 8 + 2 * t], sacc[g * 8 + 2 * t + 1], moff, ls);
    const u32x4 v4 = {pk[0], pk[1], pk[2], pk[3]};
    return __builtin_bit_cast(bf16x8, v4);
  };

  lds_u8* const kl0 = (lds_u8*)k_lds0;
  lds_u8* const kl1 = (lds_u8*)k_lds1;
  lds_u8* const vl0 = (lds_u8*)v_lds0;
  lds_u8* const vl1 = (lds_u8*)v_lds1;

  // threshold rescale of the running state for a step whose row maximum is mcur;
  // returns the exponent offset of the step's exponentials
  auto rescale = [&](float mcur, int k0) -> float {
    const float m_new = __builtin_fmaxf(m_used, mcur);
    const bool need = m_new > m_used + tau;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? exp2_(m_used - m_new) : 1.f;
      m_used = need ? m_new : m_used;
      if constexpr (COUNT) nres += need ? 1 : 0;
      l_sum *= alpha;
      if constexpr (PV != 0) lq_sum *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
    }
    // m_used is -inf only while every key seen so far is hidden (then p = 0 whatever
    // the offset)
    float moff = m_used == ninf ? 0.f : m_used;
    if constexpr (MODE == kAlibiCausal) moff = __builtin_fmaf(-slope2, (float)(k0 + 4 * hh - qrow), moff);
    if constexpr (FP8) moff -= lvs;  // P in units of vs_kb / vs_max
    return moff;
  };
  // O^T += V^T P^T: bf16 operands, or fp16 ones for fp8 inputs (the fragments carry the
  // 16-bit patterns either way)
  auto pv_mma = [&](bf16x8 va, bf16x8 pb, const f32x16& acc) -> f32x16 {
    if constexpr (FP8)
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, va), __builtin_bit_cast(f16x8, pb), acc,
                                                    0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, acc, 0, 0, 0);
  };
  // ---- the fp8/fp4 P.V (PV != 0) ---------------------------------------------------------------
  // P of a whole step as the B operand of the f8f6f4 MFMA: the lane's 32 exponentials in
  // accumulator order (j = 16 bk + r), offset moff (linear scores), V-scale units as above.
  auto p8_exp = [&](const f32x16 (&sacc)[2], int j, float moff) -> float {
    return exp2_(__builtin_fmaf(sacc[j >> 4][j & 15], ct, -moff));
  };
  // Rounds the 32 values of p to the operand's format and adds the rounded values to lq;
  // sc is the lane's E8M0 block scale byte (127 = 1 for e4m3).
  auto p8_pack = [&](const float (&p)[32], float& lq, int& sc) -> i32x8 {
    i32x8 b = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (PV == kPvE4m3) {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(p[4 * w], p[4 * w + 1], 0, false);  // round to nearest even
        x = __builtin_amdgcn_cvt_pk_fp8_f32(p[4 * w + 2], p[4 * w + 3], x, true);
        b[w] = x;
        const f32x2 d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x, 1.f, false);
        const f32x2 d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x, 1.f, true);
        lq += (d0[0] + d0[1]) + (d1[0] + d1[1]);
      }
      sc = 127;
    } else {
      // block scale 2^e: the smallest power of two with max p <= 6 * 2^e (6 = E2M1's
      // largest value), e in [-126, 127]; the codes are those of p / 2^e, nearest even
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) amax = __builtin_fmaxf(amax, p[j]);
      const uint32_t tb = __builtin_bit_cast(uint32_t, amax * (1.f / 6.f));
      int e = (int)((tb >> 23) & 255u) - 127 + ((tb & 0x7FFFFFu) != 0u ? 1 : 0);
      e = min(max(e, -126), 127);
      float sv = __builtin_ldexpf(1.f, e);
      if (amax > 6.f * sv && e < 127) {  // (amax / 6 rounded down onto a power of two)
        ++e;
        sv *= 2.f;
      } else if (e > -126 && amax <= 3.f * sv) {
        --e;
        sv *= 0.5f;
      }
      static_for<16>([&](auto tc) {  // (the byte select is an immediate)
        constexpr int t = decltype(tc)::value;
        b[t >> 2] = (int)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32((unsigned)b[t >> 2], p[2 * t], p[2 * t + 1], sv, t & 3);
      });
      static_for<16>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        const f32x2 dv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((unsigned)b[t >> 2], sv, t & 3);
        lq += dv[0] + dv[1];
      });
      sc = e + 127;
    }
    return b;
  };
  auto pv8_mma = [&](const i32x8& va, const i32x8& pb, int sc, const f32x16& acc) -> f32x16 {
    if constexpr (PV == kPvFp4)  // A e4m3 (format 0), B E2M1 (format 4) with the lane's block scale
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, acc, 0, 4, 0, 127, 0, sc);
    else
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, acc, 0, 0, 0, 127, 0, 127);
  };
  // a whole step's P.V, not pipelined (the PARTIAL tail block and the last step)
  auto pv8_step = [&](const lds_u8* vt, const f32x16 (&sacc)[2], float moff, float& ls, float& lq) {
    float p[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      p[j] = p8_exp(sacc, j, moff);
      ls += p[j];
    }
    int sc = 127;
    const i32x8 pb = p8_pack(p, lq, sc);
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = pv8_mma(vfrag8(vt, db), pb, sc, oacc[db]);
  };

  constexpr int NQ = 2 * NQC, NP = 4 * NDB, NS = NQ + NP;  // MFMAs of S = K Q^T, of O += V P, of a step
  constexpr int PD = 3;                                     // LDS fragments are read PD MFMAs ahead

  // Non-pipelined step halves (PARTIAL steps): S = K Q^T, and O += V P with the P
  // slices formed under the MFMAs of the slice before; both read their LDS fragments
  // PD MFMAs ahead, with scheduling fences between the MFMAs.
  auto qk_sched = [&](const lds_u8* kt, f32x16 (&sacc)[2]) {
    KF fr[PD + 1];
    static_for<PD>([&](auto ic) { fr[ic.value] = kfrag(kt, ic.value & 1, ic.value >> 1); });
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
    __builtin_amdgcn_sched_barrier(0);
    static_for<NQ>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i + PD < NQ) fr[(i + PD) % (PD + 1)] = kfrag(kt, (i + PD) & 1, (i + PD) >> 1);
      sacc[i & 1] = qk_mma(fr[i % (PD + 1)], qf[i >> 1], sacc[i & 1]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto pv_sched = [&](auto raw_tag, const lds_u8* vt, const f32x16 (&sacc)[2], float moff, float& ls) {
    bf16x8 fr[PD + 1], pf[4];
    static_for<PD>([&](auto ic) { fr[ic.value] = vfrag(vt, ic.value / NDB, ic.value % NDB); });
    pf[0] = pslice(raw_tag, sacc[0], 0, moff, ls);
    __builtin_amdgcn_sched_barrier(0);
    static_for<NP>([&](auto jc) {
      constexpr int j = decltype(jc)::value, ks = j / NDB, db = j % NDB;
      if constexpr (j + PD < NP) fr[(j + PD) % (PD + 1)] = vfrag(vt, (j + PD) / NDB, (j + PD) % NDB);
      oacc[db] = pv_mma(fr[j % (PD + 1)], pf[ks], oacc[db]);
      if constexpr (db == 0 && ks + 1 < 4) pf[ks + 1] = pslice(raw_tag, sacc[(ks + 1) >> 1], (ks + 1) & 1, moff, ls);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto qk_full = [&](const lds_u8* kt, f32x16 (&sacc)[2]) {
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      sacc[bk] = f32x16{};
#pragma unroll
      for (int c = 0; c < NQC; ++c)
        sacc[bk] = qk_mma(kfrag(kt, bk, c), qf[c], sacc[bk]);
    }
  };
  auto pv_full = [&](const lds_u8* vt, const bf16x8 (&pf)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = pv_mma(vfrag(vt, ks, db), pf[ks], oacc[db]);
  };

  f32x16 sa[2], sb[2];
  bf16x8 pf[4];
  constexpr std::true_type YES{};
  constexpr std::false_type NO{};

  // ---- phase 1: PARTIAL blocks, one step at a time (K(s), V(s) in buffers s % 2) ----------
  // (fp8: on entry to step s the tiles of step s are committed and those of step s+1
  // staged)
  const int np_steps = 2 * npart;
  if (nsteps > 0) {
    if constexpr (DIRECT_K) {
      issue_k(step_k0_first(0), kl0);
    } else {
      stage_k(step_k0_first(0));
      commit_k(kl0);
      if (1 < nsteps) stage_k(step_k0_first(1));
    }
    if constexpr (DIRECT_V) {
      issue_v(step_k0_first(0), vl0);
    } else {
      stage_v(step_k0_first(0));
      commit_v(vl0);
      if (1 < nsteps) stage_v(step_k0_first(1));
    }
  }
  for (int s = 0; s < np_steps; ++s) {
    lds_u8* const kc = (s & 1) ? kl1 : kl0;
    lds_u8* const vc = (s & 1) ? vl1 : vl0;
    wait_tiles();
    __syncthreads();  // K(s), V(s) in; every read of step s-1 done
    if (s + 1 < nsteps) {
      if constexpr (DIRECT_K) {
        issue_k(step_k0_first(s + 1), (s & 1) ? kl0 : kl1);
      } else {
        commit_k((s & 1) ? kl0 : kl1);
        if (s + 2 < nsteps) stage_k(step_k0(s + 2));
      }
      if constexpr (DIRECT_V) {
        issue_v(step_k0_first(s + 1), (s & 1) ? vl0 : vl1);
      } else {
        commit_v((s & 1) ? vl0 : vl1);
        if (s + 2 < nsteps) stage_v(step_k0(s + 2));
      }
    }
    const int k0 = step_k0(s);
    // A wave none of whose rows sees a key of this step skips its arithmetic: its scores
    // would all be hidden, p = 0, and the running state would stay as it is.
    if (__builtin_amdgcn_ballot_w64(lo_q <= k0 + 63 && hi_q >= k0) == 0) continue;
    scales_p(k0);
    scales_e(k0);
    qk_sched(kc, sa);
    const float moff = rescale(prepare(YES, NO, sa, k0), k0);
    float ls = 0.f;
    if constexpr (PV != 0) {
      float lq = 0.f;
      pv8_step(vc, sa, moff, ls, lq);
      lq_sum += lq * ivs;
    } else {
      pv_sched(NO, vc, sa, moff, ls);
    }
    l_sum += FP8 ? ls * ivs : ls;
  }

  // ---- phase 2: FULL blocks, software-pipelined ---------------------------------------------
  // Step s (even steps: buffers 0 -> 1 and S in sa -> sb; odd steps the reverse).  On
  // entry: S(s) in scur, prepared (softcap scores raw), with its row maximum mcur; K(s+1)
  // and V(s) requested.
  //   wait for this wave's loads, barrier (all loads in; all reads of step s-1 done);
  //   NS issue slots, one MFMA each: slots [0, NQ) S(s+1) = K(s+1) Q^T, slots
  //   [NQ, NS) O += V(s) P(s).  Every LDS fragment is read PD slots before its MFMA.
  //   The loads of the step and its rescale follow the first E slots.  The 16
  //   exponential pairs of P(s) start in slots [E, WP), pair k in slot E + k(WP-E)/16,
  //   its later stages one and two slots on, each packed before the P.V MFMA that
  //   consumes it; the transform and maximum of
  //   S(s+1) take slots [PS, NS), after its MFMAs have completed.  Scheduling fences
  //   between the slots keep this interleaving, so the VALU work of a slot runs under
  //   that slot's MFMA.  (With the e4m3 Q.K^T a step has only NQ = 2*D/64 Q.K^T MFMAs, each
  //   of twice the work: the loads and rescale follow the first slot or none, and the
  //   exponentials are packed closer so that slice 0 is ready for the first P.V MFMA.)
  constexpr int E = QK8 ? (D == 128 ? 1 : 0) : 2;  // slots issued before the loads and the rescale
  constexpr int WP = QK8 ? (D == 128 ? 11 : 5) : NQ + NP / 2;
  constexpr int PS = QK8 ? (D == 128 ? 8 : 4) : WP;  // first slot of the maximum of S(s+1)
  constexpr bool PRE = MODE == kSoftcap;  // softcap scores reach the loop raw
  constexpr int NSTG = PRE ? 3 : 2;       // slots a pair's stages span
  static_assert(PS >= NQ && PS < NS, "maximum slots");
  // pair k starts in slot E + k(WP - E)/16
  static_assert(E + ((4 * 0 + 3) * (WP - E)) / 16 + NSTG - 1 < NQ + NDB * 0 &&
                    E + ((4 * 1 + 3) * (WP - E)) / 16 + NSTG - 1 < NQ + NDB * 1 &&
                    E + ((4 * 2 + 3) * (WP - E)) / 16 + NSTG - 1 < NQ + NDB * 2 &&
                    E + ((4 * 3 + 3) * (WP - E)) / 16 + NSTG - 1 < NQ + NDB * 3,
                "every P slice is packed before its first P.V MFMA");
  auto step = [&](auto next_tag, auto issue_k_tag, int s, lds_u8* kcur, lds_u8* knext, lds_u8* vcur,
                  lds_u8* vnext, f32x16 (&scur)[2], f32x16 (&snext)[2], float& mcur) {
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr bool ISSUE_K = decltype(issue_k_tag)::value;
    wait_tiles();
    __syncthreads();
    // the loads of this step and the rescale go after the first E slots, so that the
    // matrix cores have work right after the barrier (fp8: K(s+2) and V(s+1) are committed
    // from the staging registers one 16-byte chunk per slot from slot E on, each tile
    // restaged -- K(s+3), V(s+2) -- after its last chunk; the last step commits nothing)
    float moff = 0.f;
    constexpr int VC0 = E + (DIRECT_K ? 0 : SCH);  // first slot of the V chunk commits
    auto fp8_tiles = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (!DIRECT_K && ISSUE_K && i >= E && i < E + SCH) {
        commit_k_chunk(kcur, i - E);
        if constexpr (i == E + SCH - 1) {
          if (s + 3 < nsteps) stage_k(step_k0(s + 3));
        }
      }
      if constexpr (!DIRECT_V && NEXT && i >= VC0 && i < VC0 + SCH) {
        commit_v_chunk(vnext, i - VC0);
        if constexpr (i == VC0 + SCH - 1) {
          if (s + 2 < nsteps) stage_v(step_k0(s + 2));
        }
      }
    };
    auto loads_and_rescale = [&]() {
      if constexpr (DIRECT_K && ISSUE_K) issue_k(step_k0(s + 2), kcur);
      if constexpr (DIRECT_V && NEXT) issue_v(step_k0(s + 1), vnext);
      scales_e(step_k0(s));
      moff = rescale(mcur, step_k0(s));
    };

    float ls = 0.f;
    if constexpr (NEXT) {
      const int k1 = step_k0(s + 1);
      const int kq1 = k1 + 4 * hh - qrow;
      scales_p(k1);
      // fragment of slot i, read PD slots ahead: K fragments (slots below NQ) and V
      // fragments in rings of their own, both indexed by the slot
      KF kr[PD + 1];
      bf16x8 vr[PD + 1];
      auto frag = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i < NQ) kr[i % (PD + 1)] = kfrag(knext, i & 1, i >> 1);
        else vr[i % (PD + 1)] = vfrag(vcur, (i - NQ) / NDB, (i - NQ) % NDB);
      };
      static_for<PD>([&](auto ic) { frag(ic); });
      snext[0] = f32x16{};
      snext[1] = f32x16{};
      uint32_t pk[16];
      float pv0[16], pv1[16];  // pair values between stages
      float mx = ninf;
      __builtin_amdgcn_sched_barrier(0);
      static_for<NS>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i == E) {
          loads_and_rescale();
          __builtin_amdgcn_sched_barrier(0);
        }
        fp8_tiles(ic);
        if constexpr (i + PD < NS) frag(std::integral_constant<int, i + PD>{});
        if constexpr (i < NQ) {
          snext[i & 1] = qk_mma(kr[i % (PD + 1)], qf[i >> 1], snext[i & 1]);
        } else {
          constexpr int j = i - NQ, ks = j / NDB, db = j % NDB;
          const u32x4 v4 = {pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
          oacc[db] = pv_mma(vr[i % (PD + 1)], __builtin_bit_cast(bf16x8, v4), oacc[db]);
        }
        // pair k: stages in slots a(k) (+1, +2), a(k) = E + k(WP - E)/16; the
        // instructions of one slot come from different pairs and do not wait on each other
        static_for<16>([&](auto kc) {
          constexpr int k = decltype(kc)::value;
          constexpr int a = E + (k * (WP - E)) / 16;
          constexpr int sl = k >> 2, r = (sl & 1) * 8 + 2 * (k & 3);
          if constexpr (a == i) {
            float s0 = scur[sl >> 1][r], s1 = scur[sl >> 1][r + 1];
            pin(s0);
            pin(s1);
            if constexpr (PRE) {
              s0 = p_pre(s0);
              s1 = p_pre(s1);
            } else {
              s0 = p_exp(s0, moff);
              s1 = p_exp(s1, moff);
            }
            pin(s0);
            pin(s1);
            pv0[k] = s0;
            pv1[k] = s1;
          }
          if constexpr (PRE && a + 1 == i) {
            pv0[k] = p_exp(pv0[k], moff);
            pv1[k] = p_exp(pv1[k], moff);
            pin(pv0[k]);
            pin(pv1[k]);
          }
          if constexpr (a + NSTG - 1 == i) {
            pk[k] = p_pack(pv0[k], pv1[k], ls);
            pin(pk[k]);
            pin(ls);
          }
        });
        if constexpr (i >= PS) {
          // S(s+1) elements [32(i - PS)/(NS - PS), 32(i - PS + 1)/(NS - PS)) in this slot
          constexpr int e0 = 32 * (i - PS) / (NS - PS), e1 = 32 * (i - PS + 1) / (NS - PS);
          static_for<e1 - e0>([&](auto ec) {
            constexpr int idx = e0 + decltype(ec)::value, bk = idx >> 4, r = idx & 15;
            float sv = snext[bk][r];
            pin(sv);
            const float x = xform(sv, bk, r, kq1);
            snext[bk][r] = x;
            mx = __builtin_fmaxf(mx, x);
          });
          pin(mx);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      mcur = finalize(mx, k1);
    } else {
      loads_and_rescale();
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) pf[sl] = pslice(YES, scur[sl >> 1], sl & 1, moff, ls);
      pv_full(vcur, pf);
    }
    l_sum += FP8 ? ls * ivs : ls;
  };

  // The fp8/fp4 P.V step: 4 Q.K^T MFMAs of S(s+1) with the 32 exponentials of P(s) under
  // them (8 per slot) and P(s) rounded to the operand after the last, then the 4 P.V MFMAs
  // (one per 32-wide d block, each taking the whole step's P) with the maximum of S(s+1).
  auto step8 = [&](auto next_tag, auto issue_k_tag, int s, lds_u8* kcur, lds_u8* knext, lds_u8* vcur,
                   lds_u8* vnext, f32x16 (&scur)[2], f32x16 (&snext)[2], float& mcur) {
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr bool ISSUE_K = decltype(issue_k_tag)::value;
    wait_tiles();
    __syncthreads();
    float moff = 0.f, ls = 0.f, lq = 0.f;
    auto loads_and_rescale = [&]() {
      if constexpr (ISSUE_K) issue_k(step_k0(s + 2), kcur);
      if constexpr (NEXT) issue_v(step_k0(s + 1), vnext);
      scales_e(step_k0(s));
      moff = rescale(mcur, step_k0(s));
    };
    if constexpr (NEXT) {
      const int k1 = step_k0(s + 1);
      scales_p(k1);
      KF kr[2];
      kr[0] = kfrag(knext, 0, 0);
      kr[1] = kfrag(knext, 1, 0);
      snext[0] = f32x16{};
      snext[1] = f32x16{};
      float p[32];
      i32x8 pb = {0, 0, 0, 0, 0, 0, 0, 0}, vf[2];
      int sc = 127;
      float mx = ninf;
      __builtin_amdgcn_sched_barrier(0);
      static_for<NQ + NDB>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i == 0) {
          loads_and_rescale();
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (i < NQ) {
          snext[i & 1] = qk_mma(kr[i & 1], qf[i >> 1], snext[i & 1]);
          if constexpr (i + 2 < NQ) kr[i & 1] = kfrag(knext, (i + 2) & 1, (i + 2) >> 1);
          static_for<32 / NQ>([&](auto jc) {
            constexpr int j = i * (32 / NQ) + decltype(jc)::value;
            p[j] = p8_exp(scur, j, moff);
            ls += p[j];
          });
          if constexpr (i == NQ - 2) vf[0] = vfrag8(vcur, 0);
          if constexpr (i == NQ - 1) {
            pb = p8_pack(p, lq, sc);
            vf[1] = vfrag8(vcur, 1);
          }
        } else {
          constexpr int db = i - NQ;
          oacc[db] = pv8_mma(vf[db & 1], pb, sc, oacc[db]);
          if constexpr (db + 2 < NDB) vf[db & 1] = vfrag8(vcur, db + 2);
          static_for<32 / NDB>([&](auto ec) {
            constexpr int idx = db * (32 / NDB) + decltype(ec)::value;
            mx = __builtin_fmaxf(mx, snext[idx >> 4][idx & 15]);
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      mcur = finalize(mx, k1);
    } else {
      loads_and_rescale();
      pv8_step(vcur, scur, moff, ls, lq);
    }
    l_sum += ls * ivs;
    lq_sum += lq * ivs;
  };
  auto run_step = [&](auto next_tag, auto issue_k_tag, int s, lds_u8* kcur, lds_u8* knext, lds_u8* vcur,
                      lds_u8* vnext, f32x16 (&scur)[2], f32x16 (&snext)[2], float& mcur) {
    if constexpr (PV != 0) step8(next_tag, issue_k_tag, s, kcur, knext, vcur, vnext, scur, snext, mcur);
    else step(next_tag, issue_k_tag, s, kcur, knext, vcur, vnext, scur, snext, mcur);
  };

  if (np_steps < nsteps) {
    const int t = np_steps;  // first FULL step (even); K(t), V(t) requested
    wait_tiles();
    __syncthreads();  // K(t) in; every read of step t-1 done
    if (t + 1 < nsteps) {
      if constexpr (DIRECT_K) {
        issue_k(step_k0_first(t + 1), kl1);
      } else {
        commit_k(kl1);
        if (t + 2 < nsteps) stage_k(step_k0(t + 2));
      }
    }
    qk_full(kl0, sa);
    scales_p(step_k0(t));
    float mcand = prepare(NO, YES, sa, step_k0(t));
    int s = t;
    for (; s + 2 < nsteps; s += 2) {
      run_step(YES, YES, s, kl0, kl1, vl0, vl1, sa, sb, mcand);
      run_step(YES, YES, s + 1, kl1, kl0, vl1, vl0, sb, sa, mcand);
    }
    run_step(YES, NO, s, kl0, kl1, vl0, vl1, sa, sb, mcand);
    run_step(NO, NO, s + 1, kl1, kl0, vl1, vl0, sb, sa, mcand);
  }

  // ---- epilogue -------------------------------------------------------------------------
  l_sum = pair_sum(l_sum);
  if constexpr (PV != 0) lq_sum = pair_sum(lq_sum);
  const float nanv = __builtin_bit_cast(float, 0x7fc00000u);  // quiet NaN (a bit pattern, not folded)
  const float onorm = PV != 0 ? lq_sum : l_sum;
  const float inv = invalid ? nanv : (onorm > 0.f ? (FP8 ? vs_max : 1.f) / onorm : 0.f);
  // O leaves through LDS, so that each store instruction writes whole rows (a lane holds
  // 8-byte pieces of one row, which would make every store touch 32 rows).  The wave's
  // 32 x D tile goes to a region of its own in K buffer 0 (waves 0, 1) or V buffer 0
  // (waves 2, 3), which no step reads any more: the step count is even, so the last step
  // reads only buffers 1, and the barrier at its start saw every read of buffers 0 done.
  // Chunk ch (16 bytes) of row r sits at chunk position ch ^ (r % CPR), its two 8-byte
  // halves swapped when (r / CPR) is odd; then the wave stores RPR whole rows per
  // instruction, 16 bytes per lane.
  {
    constexpr int RPR = 64 / CPR;  // rows per 1 KiB store
    lds_u8* const ot = (wave < 2 ? kl0 : vl0) + (wave & 1) * (32 * ROWB);
    const int wsw = (l32 / CPR) & 1;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x2 v01 = to_bf16x2(oacc[db][4 * i + 0] * inv, oacc[db][4 * i + 1] * inv);
        const bf16x2 v23 = to_bf16x2(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
        const u32x2 st = {__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23)};
        const int pos = (4 * db + i) ^ (l32 % CPR);  // chunk of d = 32 db + 8 i + 4 hh
        *(__attribute__((address_space(3))) u32x2*)(ot + l32 * ROWB + pos * 16 + 8 * (hh ^ wsw)) = st;
      }
    const int rl = lane / CPR, ch = lane % CPR;
    bf16* const orow0 = (bf16*)a.o + (head_row0 + q0 + wave * 32) * D;
#pragma unroll
    for (int k = 0; k < 32 / RPR; ++k) {
      const int r = RPR * k + rl;
      u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(ot + r * ROWB + ((ch ^ (r % CPR)) * 16));
      if (((RPR * k) / CPR) & 1) v = u32x4{v.z, v.w, v.x, v.y};  // (the swapped halves)
      if (q0 + wave * 32 + r < N) *(u32x4*)(orow0 + r * D + ch * 8) = v;
    }
  }
  if (qvalid && hh == 0) {
    float lse;
    if (invalid) lse = nanv;
    else if (l_sum > 0.f) lse = (m_used + __builtin_amdgcn_logf(l_sum)) * 0.6931471805599453f;
    else lse = ninf;
    a.lse[head_row0 + qrow] = lse;
    if constexpr (COUNT) a.rescale_counts[head_row0 + qrow] = nres;
  }
}

// Launches the variant (masked, mode, generic modifiers) chosen on the host; a
// document mask is never launched without a block map (causal and window masks may
// come without one: the kernel derives their lists).  With the e4m3 Q.K^T (QK8) a
// softcap without ALiBi runs in the generic mode (its transform before the maximum).
template <int D, bool FP8, bool QK8, bool COUNT, int PV>
hipError_t launch(const FwdArgs& a, bool masked, int mode, bool galibi, bool gsoftcap, hipStream_t st) {
  if (COUNT != (a.rescale_counts != nullptr)) return hipErrorInvalidValue;
  if constexpr (PV != 0) {
    // the fp8/fp4 P.V: e4m3 inputs and Q.K^T, no positional mask, linear scores
    const dim3 grid((unsigned)(a.B * a.H * a.nqb)), block(256);
    if (masked || mode != kLinear || !a.q_scale || !a.k_scale || !a.v_scale) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true, true, false, PV, false, kLinear, false, false>), grid, block, 0,
                       st, a);
    return hipGetLastError();
  } else {
  const dim3 grid((unsigned)(a.B * a.H * a.nqb)), block(256);
  if (masked && a.map == nullptr && (a.mflags & kDocument)) return hipErrorInvalidValue;
  if (FP8 && (!a.q_scale || !a.k_scale || !a.v_scale)) return hipErrorInvalidValue;
  if (QK8 && mode == kSoftcap) {
    mode = kGeneric;
    galibi = false;
    gsoftcap = true;
  }
  constexpr int kSC = QK8 ? kGeneric : kSoftcap;   // the softcap-only mode
  constexpr bool kSCA = false, kSCS = QK8;         // its generic modifiers
  const bool softcap_only = QK8 ? (mode == kGeneric && !galibi && gsoftcap) : mode == kSoftcap;
  if (masked) {
    if (mode == kLinear) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, FP8, QK8, COUNT, 0, true, kLinear, false, false>), grid, block, 0, st, a);
    else if (softcap_only) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, FP8, QK8, COUNT, 0, true, kSC, kSCA, kSCS>), grid, block, 0, st, a);
    else if (mode == kAlibiCausal) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, FP8, QK8, COUNT, 0, true, kAlibiCausal, false, false>), grid, block, 0, st, a);
    else if (mode == kGeneric && galibi && !gsoftcap) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, FP8, QK8, COUNT, 0, true, kGeneric, true, false>), grid, block, 0, st, a);
    else if (mode == kGeneric && galibi && gsoftcap) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, FP8, QK8, COUNT, 0, true, kGeneric, true, true>), grid, block, 0, st, a);
    else return hipErrorInvalidValue;
  } else {
    if (mode == kLinear) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, FP8, QK8, COUNT, 0, false, kLinear, false, false>), grid, block, 0, st, a);
    else if (softcap_only) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, FP8, QK8, COUNT, 0, false, kSC, kSCA, kSCS>), grid, block, 0, st, a);
    else if (mode == kGeneric && galibi && !gsoftcap) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, FP8, QK8, COUNT, 0, false, kGeneric, true, false>), grid, block, 0, st, a);
    else if (mode == kGeneric && galibi && gsoftcap) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, FP8, QK8, COUNT, 0, false, kGeneric, true, true>), grid, block, 0, st, a);
    else return hipErrorInvalidValue;  // (ALiBi on a causal mask always has a block map)
  }
  return hipGetLastError();
  }
}

}  // namespace bf16path
}  // namespace attn119
