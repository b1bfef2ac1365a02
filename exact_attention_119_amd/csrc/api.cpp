// C ABI of libattn119.so: argument validation, block-map entry points and the
// dispatch of the forward pass to its compiled variants.  Declarations and the
// full contract are in include/attn119.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/attn119.h"
#include "common.hpp"
#include "fwd_args.hpp"

namespace attn119 {
hipError_t launch_blockmap(unsigned char* map, int B, int N, uint32_t flags, int window,
                           const int32_t* doc_id, const int32_t* cu, int nseq, int32_t* ids, bool compact,
                           hipStream_t stream);
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv, float* delta, int B, int H, int Hkv, int N, int d, float scale,
                      uint32_t flags, int window, float softcap, const float* slopes, const void* map,
                      hipStream_t stream, bool compact_map);
hipError_t launch_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                              float scale, uint32_t flags, int window, float softcap, const float* slopes,
                              const void* map, hipStream_t stream, bool compact_map);
size_t bwd_scratch_rows();
hipError_t launch_quant(const void* x, void* codes, float* scales, int BH, int N, int d, const uint32_t* signs,
                        hipStream_t stream);
constexpr int kInBf16 = 0, kInFp8 = 1, kInFp8Qk8 = 2, kInFp8Pv8 = 3, kInFp8Pv4 = 4;
namespace bf16path {
constexpr int kLinear = 0, kSoftcap = 1, kAlibiCausal = 2, kGeneric = 3;
constexpr int kPvE4m3 = 1, kPvFp4 = 2;
template <int D, bool FP8, bool QK8, bool COUNT, int PV>
hipError_t launch(const FwdArgs& a, bool masked, int mode, bool galibi, bool gsoftcap, hipStream_t st);
}  // namespace bf16path
}  // namespace attn119

using namespace attn119;

namespace {

constexpr double kLog2e = 1.4426950408889634;
constexpr uint32_t kAllFlags = ATTN_CAUSAL | ATTN_WINDOW | ATTN_DOCUMENT | ATTN_ALIBI | ATTN_SOFTCAP;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool positional(const attn_mask* m) { return m && (m->flags & (ATTN_CAUSAL | ATTN_WINDOW | ATTN_DOCUMENT)); }

// The compiled kernel variant a call selects (host logic only, testable on a CPU).
struct FwdVariant {
  int d;
  int input;     // kInBf16, kInFp8, kInFp8Qk8, kInFp8Pv8, kInFp8Pv4
  bool masked;   // positional mask through the block map
  int mode;      // bf16 kernel: score-modifier mode
  bool alibi, softcap;
};

FwdVariant select_variant(int32_t d, int32_t dtype, const attn_mask* mask, const attn_fp8* fp8) {
  FwdVariant v;
  const uint32_t flags = mask ? mask->flags : 0u;
  v.d = d;
  v.input = dtype == ATTN_BF16 ? kInBf16 : (fp8 && fp8->qk_mode == ATTN_QK_E4M3 ? kInFp8Qk8 : kInFp8);
  if (v.input == kInFp8Qk8 && fp8->pv_mode == ATTN_PV_E4M3) v.input = kInFp8Pv8;
  if (v.input == kInFp8Qk8 && fp8->pv_mode == ATTN_PV_FP4) v.input = kInFp8Pv4;
  v.masked = positional(mask);
  v.alibi = flags & ATTN_ALIBI;
  v.softcap = flags & ATTN_SOFTCAP;
  if (!v.alibi) v.mode = v.softcap ? bf16path::kSoftcap : bf16path::kLinear;
  else if (!v.softcap && (flags & ATTN_CAUSAL)) v.mode = bf16path::kAlibiCausal;
  else v.mode = bf16path::kGeneric;
  return v;
}

// Table of variant names, built once.  A function-local static is initialised exactly
// once even under concurrent first calls (C++11), so every caller sees it complete.
struct VariantNames {
  char names[2][5][2][5][64];
  VariantNames() {
    static const char* const kIn[] = {"bf16", "fp8", "fp8-qk8", "fp8-qk8-pv8", "fp8-qk8-pv4"};
    static const char* const kMode[] = {"linear", "softcap", "alibi-causal", "generic-alibi",
                                        "generic-alibi-softcap"};
    for (int di = 0; di < 2; ++di)
      for (int in = 0; in < 5; ++in)
        for (int m = 0; m < 2; ++m)
          for (int k = 0; k < 5; ++k)
            std::snprintf(names[di][in][m][k], 64, "%s d%d %s %s", kIn[in], di ? 128 : 64,
                          m ? "masked" : "unmasked", kMode[k]);
  }
};

const char* variant_name(const FwdVariant& v) {
  static const VariantNames table;
  const auto& names = table.names;
  const int k = v.mode == bf16path::kGeneric ? (v.softcap ? 4 : 3) : v.mode;
  return names[v.d == 128][v.input][v.masked][k];
}

attn_status check_mask(const attn_mask* m) {
  if (!m) return ATTN_OK;
  if (m->flags & ~kAllFlags) return ATTN_ERR_UNSUPPORTED;
  if ((m->flags & ATTN_WINDOW) && m->window < 1) return ATTN_ERR_INVALID_ARG;
  if (m->flags & ATTN_SOFTCAP) {
    if (!(m->softcap > 0.f) || !std::isfinite(m->softcap)) return ATTN_ERR_INVALID_ARG;
  }
  if ((m->flags & ATTN_DOCUMENT) && !m->doc_id) return ATTN_ERR_INVALID_ARG;
  if (m->doc_id && !aligned16(m->doc_id) && (m->flags & ATTN_DOCUMENT)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

attn_status check_shape(int32_t B, int32_t N) {
  if (B < 1 || N < 1) return ATTN_ERR_INVALID_ARG;
  // every int offset the kernels form must stay below 2^31
  const int64_t nb = (N + 127) / 128;
  if ((int64_t)B * N > (int64_t)INT32_MAX || (int64_t)B * nb * nb > (int64_t)INT32_MAX)
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// Offsets of the block map of (B, N): the general form or the compact one (no class and
// list sections).
attn_status layout_of(int32_t B, int32_t N, bool compact, attn_blockmap_layout* layout) {
  if (!layout) return ATTN_ERR_INVALID_ARG;
  const attn_status st = check_shape(B, N);
  if (st != ATTN_OK) return st;
  const MapLayout m = map_layout(B, N, compact);
  layout->cls = m.cls;
  layout->counts = m.counts;
  layout->idx = m.idx;
  layout->row_lo = m.row_lo;
  layout->row_hi = m.row_hi;
  layout->col_lo = m.col_lo;
  layout->col_hi = m.col_hi;
  layout->pairs = m.pairs;
  layout->status = m.status;
  layout->order = m.order;
  layout->total = m.total;
  return ATTN_OK;
}

attn_status map_bytes(int32_t B, int32_t N, const attn_mask* mask, bool compact, size_t* bytes) {
  if (!bytes) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_shape(B, N);
  if (st != ATTN_OK) return st;
  st = check_mask(mask);
  if (st != ATTN_OK) return st;
  *bytes = map_layout(B, N, compact).total;
  return ATTN_OK;
}

attn_status build_map(int32_t B, int32_t N, const attn_mask* mask, void* map, size_t bytes, bool compact,
                      void* stream) {
  size_t need = 0;
  attn_status st = map_bytes(B, N, mask, compact, &need);
  if (st != ATTN_OK) return st;
  if (!map || !aligned16(map)) return ATTN_ERR_INVALID_ARG;
  if (bytes != need) return ATTN_ERR_BAD_BLOCKMAP;
  const uint32_t flags = mask ? mask->flags : 0u;
  const int window = (mask && (flags & ATTN_WINDOW)) ? mask->window : 0;
  const int32_t* doc = (mask && (flags & ATTN_DOCUMENT)) ? mask->doc_id : nullptr;
  if (launch_blockmap((unsigned char*)map, B, N, flags, window, doc, nullptr, 0, nullptr, compact,
                      (hipStream_t)stream) !=
      hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

// The form of a block map of (B, N) passed with `bytes` bytes: the compact one when the
// size is the compact layout's (the general layout is always larger).
bool compact_form(int32_t B, int32_t N, size_t bytes) { return bytes == map_layout(B, N, true).total; }

// Variable-length workspace: the compact block map of (B = 1, N = total), then the doc ids.
size_t varlen_doc_offset(int32_t total) { return map_layout(1, total, true).total; }
size_t varlen_bytes(int32_t total) { return varlen_doc_offset(total) + align256((size_t)total * 4); }

attn_status check_varlen_mask(const attn_mask* mask) {
  const attn_status st = check_mask(mask);
  if (st != ATTN_OK) return st;
  if (mask && (mask->flags & ATTN_DOCUMENT)) return ATTN_ERR_INVALID_ARG;  // the sequences are the documents
  return ATTN_OK;
}

// The mask a variable-length call runs with: the caller's flags plus the document mask
// over the workspace's doc ids.
attn_mask varlen_mask(const attn_mask* mask, const void* workspace, int32_t total) {
  attn_mask m;
  std::memset(&m, 0, sizeof(m));
  if (mask) m = *mask;
  m.flags |= ATTN_DOCUMENT;
  m.doc_id = (const int32_t*)((const unsigned char*)workspace + varlen_doc_offset(total));
  return m;
}

}  // namespace

extern "C" {

const char* attn_status_str(int32_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dim, dtype, flag or pv mode";
    case ATTN_ERR_BAD_BLOCKMAP: return "block map missing or of the wrong size";
    case ATTN_ERR_HIP: return "HIP runtime error";
    case ATTN_ERR_BAD_DOC_ID: return "doc_id decreases (documents must be contiguous)";
    default: return "unknown status";
  }
}

attn_status attn_blockmap_layout_of(int32_t B, int32_t N, attn_blockmap_layout* layout) {
  return layout_of(B, N, false, layout);
}

attn_status attn_blockmap_compact_layout_of(int32_t B, int32_t N, attn_blockmap_layout* layout) {
  return layout_of(B, N, true, layout);
}

attn_status attn_blockmap_bytes(int32_t B, int32_t N, const attn_mask* mask, size_t* bytes) {
  return map_bytes(B, N, mask, false, bytes);
}

attn_status attn_blockmap_compact_bytes(int32_t B, int32_t N, const attn_mask* mask, size_t* bytes) {
  return map_bytes(B, N, mask, true, bytes);
}

attn_status attn_blockmap_build(int32_t B, int32_t N, const attn_mask* mask, void* map, size_t bytes,
                                void* stream) {
  return build_map(B, N, mask, map, bytes, false, stream);
}

attn_status attn_blockmap_build_compact(int32_t B, int32_t N, const attn_mask* mask, void* map, size_t bytes,
                                        void* stream) {
  return build_map(B, N, mask, map, bytes, true, stream);
}

attn_status attn_blockmap_status(const void* map, size_t bytes, void* stream) {
  if (!map || bytes < 256) return ATTN_ERR_INVALID_ARG;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return ATTN_ERR_HIP;
  MapHeader hd;
  if (hipMemcpy(&hd, map, sizeof(hd), hipMemcpyDeviceToHost) != hipSuccess) return ATTN_ERR_HIP;
  if (hd.magic != kMapMagic || check_shape(hd.B, hd.N) != ATTN_OK) return ATTN_ERR_BAD_BLOCKMAP;
  if (hd.compact != 0 && hd.compact != 1) return ATTN_ERR_BAD_BLOCKMAP;
  const MapLayout m = map_layout(hd.B, hd.N, hd.compact != 0);
  // a packed batch's compact map may come with the rest of its workspace
  if (bytes != m.total && !(hd.compact && hd.B == 1 && bytes == varlen_bytes(hd.N))) return ATTN_ERR_BAD_BLOCKMAP;
  const size_t n = (size_t)hd.B * hd.nqb;
  int32_t* st = new int32_t[n];
  const hipError_t e = hipMemcpy(st, (const unsigned char*)map + m.status, n * 4, hipMemcpyDeviceToHost);
  int bad = 0;
  for (size_t i = 0; i < n; ++i) bad |= st[i];
  delete[] st;
  if (e != hipSuccess) return ATTN_ERR_HIP;
  return bad ? ATTN_ERR_BAD_DOC_ID : ATTN_OK;
}

attn_status attn_check_args_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B,
                                int32_t H, int32_t H_kv, int32_t N, int32_t d, float scale, int32_t dtype,
                                const attn_mask* mask, const void* blockmap, size_t blockmap_bytes,
                                const attn_fp8* fp8, float rescale_tau) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (H < 1 || H_kv < 1 || H % H_kv != 0) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_shape(B, N);
  if (st != ATTN_OK) return st;
  if ((int64_t)B * H > (int64_t)INT32_MAX / ((N + 127) / 128) ||
      (int64_t)B * H * N > (int64_t)INT32_MAX * 8)
    return ATTN_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (!(rescale_tau >= 0.f && rescale_tau <= 8.f)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
  st = check_mask(mask);
  if (st != ATTN_OK) return st;
  if (mask && (mask->flags & ATTN_ALIBI) && mask->alibi_slopes && !aligned16(mask->alibi_slopes))
    return ATTN_ERR_INVALID_ARG;
  if (dtype == ATTN_FP8_E4M3) {
    if (!fp8 || !fp8->q_scale || !fp8->k_scale || !fp8->v_scale) return ATTN_ERR_INVALID_ARG;
    if (fp8->qk_mode != ATTN_QK_BF16 && fp8->qk_mode != ATTN_QK_E4M3) return ATTN_ERR_UNSUPPORTED;
    if (fp8->pv_mode != ATTN_PV_F16 && fp8->pv_mode != ATTN_PV_E4M3 && fp8->pv_mode != ATTN_PV_FP4)
      return ATTN_ERR_UNSUPPORTED;
    // the fp8/fp4 P.V: with the e4m3 Q.K^T, d = 128, no mask and no score modifier
    if (fp8->pv_mode != ATTN_PV_F16 &&
        (fp8->qk_mode != ATTN_QK_E4M3 || d != 128 || (mask && mask->flags != 0u)))
      return ATTN_ERR_UNSUPPORTED;
  }
  if (positional(mask)) {
    // Causal and window masks may come without a map (the kernel derives the block lists
    // from the flags); a document mask needs one.
    const bool need = (mask->flags & ATTN_DOCUMENT) != 0;
    if (blockmap || need) {
      if (!blockmap || !aligned16(blockmap)) return ATTN_ERR_BAD_BLOCKMAP;
      // either form of the map (told apart by its size)
      if (blockmap_bytes != map_layout(B, N).total && !compact_form(B, N, blockmap_bytes))
        return ATTN_ERR_BAD_BLOCKMAP;
    }
  }
  return ATTN_OK;
}

attn_status attn_check_args(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B,
                            int32_t H, int32_t N, int32_t d, float scale, int32_t dtype,
                            const attn_mask* mask, const void* blockmap, size_t blockmap_bytes,
                            const attn_fp8* fp8, float rescale_tau) {
  return attn_check_args_gqa(q, k, v, o, lse, B, H, H, N, d, scale, dtype, mask, blockmap, blockmap_bytes,
                             fp8, rescale_tau);
}

const char* attn_fwd_kernel_name(int32_t d, int32_t dtype, const attn_mask* mask, const attn_fp8* fp8) {
  if (d != 64 && d != 128) return nullptr;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return nullptr;
  if (check_mask(mask) != ATTN_OK) return nullptr;
  if (dtype == ATTN_FP8_E4M3 && !fp8) return nullptr;
  return variant_name(select_variant(d, dtype, mask, fp8));
}

}  // extern "C"

namespace {

// The forward pass behind attn_fwd_gqa and attn_fwd_rescale_counts (counts: null, or
// device int32 [B][H][N] for the rescale events of every query row).
attn_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B, int32_t H,
                     int32_t H_kv, int32_t N, int32_t d, float scale, int32_t dtype, const attn_mask* mask,
                     const void* blockmap, size_t blockmap_bytes, const attn_fp8* fp8, float rescale_tau,
                     int32_t* counts, void* stream) {
  const attn_status st = attn_check_args_gqa(q, k, v, o, lse, B, H, H_kv, N, d, scale, dtype, mask, blockmap,
                                             blockmap_bytes, fp8, rescale_tau);
  if (st != ATTN_OK) return st;
  const uint32_t flags = mask ? mask->flags : 0u;
  const bool masked = positional(mask);
  const bool alibi = flags & ATTN_ALIBI;
  const bool softcap = flags & ATTN_SOFTCAP;

  FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = H_kv;
  a.N = N;
  a.nqb = (N + 127) / 128;
  a.c = (float)((double)scale * kLog2e);
  if (softcap) {
    a.sc2 = (float)(2.0 * (double)scale * kLog2e / (double)mask->softcap);
    a.cap2 = (float)((double)mask->softcap * kLog2e);
  }
  a.tau = rescale_tau;
  a.rescale_counts = counts;
  a.alibi_exp = (float)(-8.0 / (double)H);
  a.alibi_slopes = (alibi && mask) ? mask->alibi_slopes : nullptr;
  if (dtype == ATTN_FP8_E4M3) {
    a.q_scale = fp8->q_scale;
    a.k_scale = fp8->k_scale;
    a.v_scale = fp8->v_scale;
  }
  if (masked) {
    a.map = (const unsigned char*)blockmap;
    const bool compact_map = compact_form(B, N, blockmap_bytes);
    a.lay = map_layout(B, N, compact_map);
    a.compact = compact_map ? 1 : 0;
    a.mflags = flags & (ATTN_CAUSAL | ATTN_WINDOW | ATTN_DOCUMENT);
    a.window = (flags & ATTN_WINDOW) ? mask->window : 0;
  }
  // Causal masks give the last row blocks of a head the most key blocks.  When the grid
  // is only a few workgroups per slot (2 per CU on 256 CUs), take them heaviest-first; with
  // grouped key/value heads (no window) also when each group stays on one XCD: that order
  // then runs all query heads of a group there at once, sharing their K/V in its L2
  // (measured 4-12% faster on four grouped-query shapes; for ungrouped heads at larger
  // grids it was not faster).
  constexpr long kSlots = 2 * 256;
  const long items = (long)B * H * a.nqb;
  // (the heaviest-first order keeps a group's query heads on one XCD only when the 8
  // XCDs take equal runs of B*H/8 consecutive heads and a group never straddles two runs)
  const long bh = (long)B * H;
  const bool group_on_xcd = bh % 8 == 0 && (bh / 8) % (H / H_kv) == 0;
  const bool grouped = H_kv < H && !(flags & ATTN_WINDOW) && group_on_xcd;
  a.order = ((flags & ATTN_CAUSAL) && (items < 4 * kSlots || grouped)) ? kOrderHeavyFirst : kOrderHeadMajor;
  // Under a document mask a row block's work depends on its place in its document: take
  // the heaviest-first order the map builder derived from the block lists.
  if (masked && (flags & ATTN_DOCUMENT)) a.order = kOrderMapSorted;
  hipError_t e;
  const hipStream_t s = (hipStream_t)stream;
  const FwdVariant var = select_variant(d, dtype, mask, fp8);
  if (counts)  // (bf16 only: checked by the entry point)
    e = d == 128 ? bf16path::launch<128, false, false, true, 0>(a, var.masked, var.mode, var.alibi, var.softcap, s)
                 : bf16path::launch<64, false, false, true, 0>(a, var.masked, var.mode, var.alibi, var.softcap, s);
  else if (dtype == ATTN_BF16)
    e = d == 128 ? bf16path::launch<128, false, false, false, 0>(a, var.masked, var.mode, var.alibi, var.softcap, s)
                 : bf16path::launch<64, false, false, false, 0>(a, var.masked, var.mode, var.alibi, var.softcap, s);
  else if (fp8->qk_mode == ATTN_QK_BF16)
    e = d == 128 ? bf16path::launch<128, true, false, false, 0>(a, var.masked, var.mode, var.alibi, var.softcap, s)
                 : bf16path::launch<64, true, false, false, 0>(a, var.masked, var.mode, var.alibi, var.softcap, s);
  else if (fp8->pv_mode == ATTN_PV_E4M3)  // (d = 128: checked)
    e = bf16path::launch<128, true, true, false, bf16path::kPvE4m3>(a, var.masked, var.mode, var.alibi, var.softcap, s);
  else if (fp8->pv_mode == ATTN_PV_FP4)
    e = bf16path::launch<128, true, true, false, bf16path::kPvFp4>(a, var.masked, var.mode, var.alibi, var.softcap, s);
  else
    e = d == 128 ? bf16path::launch<128, true, true, false, 0>(a, var.masked, var.mode, var.alibi, var.softcap, s)
                 : bf16path::launch<64, true, true, false, 0>(a, var.masked, var.mode, var.alibi, var.softcap, s);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

attn_status attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B,
                         int32_t H, int32_t H_kv, int32_t N, int32_t d, float scale, int32_t dtype,
                         const attn_mask* mask, const void* blockmap, size_t blockmap_bytes, const attn_fp8* fp8,
                         float rescale_tau, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, H_kv, N, d, scale, dtype, mask, blockmap, blockmap_bytes, fp8,
                  rescale_tau, nullptr, stream);
}

attn_status attn_fwd_rescale_counts(const void* q, const void* k, const void* v, void* o, float* lse,
                                    int32_t* counts, int32_t B, int32_t H, int32_t H_kv, int32_t N, int32_t d,
                                    float scale, int32_t dtype, const attn_mask* mask, const void* blockmap,
                                    size_t blockmap_bytes, const attn_fp8* fp8, float rescale_tau, void* stream) {
  if (!counts || (reinterpret_cast<uintptr_t>(counts) & 3u)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;  // the counting kernels are built for bf16 inputs
  return fwd_impl(q, k, v, o, lse, B, H, H_kv, N, d, scale, dtype, mask, blockmap, blockmap_bytes, fp8,
                  rescale_tau, counts, stream);
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B, int32_t H,
                     int32_t N, int32_t d, float scale, int32_t dtype, const attn_mask* mask,
                     const void* blockmap, size_t blockmap_bytes, const attn_fp8* fp8, float rescale_tau,
                     void* stream) {
  return attn_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, scale, dtype, mask, blockmap, blockmap_bytes, fp8,
                      rescale_tau, stream);
}

attn_status attn_varlen_workspace_bytes(int32_t total, const attn_mask* mask, size_t* bytes) {
  if (!bytes) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_shape(1, total);
  if (st != ATTN_OK) return st;
  st = check_varlen_mask(mask);
  if (st != ATTN_OK) return st;
  *bytes = varlen_bytes(total);
  return ATTN_OK;
}

attn_status attn_varlen_prepare(const int32_t* cu_seqlens, int32_t nseq, int32_t total, const attn_mask* mask,
                                void* workspace, size_t bytes, void* stream) {
  size_t need = 0;
  const attn_status st = attn_varlen_workspace_bytes(total, mask, &need);
  if (st != ATTN_OK) return st;
  if (!cu_seqlens || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) || nseq < 1 || nseq == INT32_MAX)
    return ATTN_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace)) return ATTN_ERR_INVALID_ARG;
  if (bytes != need) return ATTN_ERR_BAD_BLOCKMAP;
  const attn_mask m = varlen_mask(mask, workspace, total);
  const hipStream_t s = (hipStream_t)stream;
  const int window = (m.flags & ATTN_WINDOW) ? m.window : 0;
  // (the map kernel writes the sequence ids as it builds the map; the work order follows
  // in a second launch)
  if (launch_blockmap((unsigned char*)workspace, 1, total, m.flags, window, nullptr, cu_seqlens, nseq,
                      (int32_t*)m.doc_id, true, s) !=
      hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, int32_t H,
                            int32_t H_kv, int32_t total, int32_t d, float scale, int32_t dtype,
                            const attn_mask* mask, const void* workspace, size_t bytes, const attn_fp8* fp8,
                            float rescale_tau, void* stream) {
  size_t need = 0;
  const attn_status st = attn_varlen_workspace_bytes(total, mask, &need);
  if (st != ATTN_OK) return st;
  if (!workspace || !aligned16(workspace)) return ATTN_ERR_INVALID_ARG;
  if (bytes != need) return ATTN_ERR_BAD_BLOCKMAP;
  const attn_mask m = varlen_mask(mask, workspace, total);
  return attn_fwd_gqa(q, k, v, o, lse, 1, H, H_kv, total, d, scale, dtype, &m, workspace,
                      varlen_doc_offset(total), fp8, rescale_tau, stream);
}

attn_status attn_varlen_layout_of(int32_t total, attn_blockmap_layout* layout) {
  return layout_of(1, total, true, layout);
}

attn_status attn_fp8_quantize(const void* x, void* codes, float* scales, int32_t B, int32_t H, int32_t N,
                              int32_t d, const uint32_t* rotate_signs, void* stream) {
  if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes) ||
      (reinterpret_cast<uintptr_t>(scales) & 3u))
    return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H * ((N + 127) / 128) > (int64_t)INT32_MAX) return ATTN_ERR_INVALID_ARG;
  if (launch_quant(x, codes, scales, B * H, N, d, rotate_signs, (hipStream_t)stream) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* delta, int32_t B, int32_t H,
                         int32_t H_kv, int32_t N, int32_t d, float scale, const attn_mask* mask,
                         const void* blockmap, size_t blockmap_bytes, void* stream) {
  attn_status st = attn_check_args_gqa(q, k, v, const_cast<void*>(o), const_cast<float*>(lse), B, H, H_kv, N, d,
                                       scale, ATTN_BF16, mask, blockmap, blockmap_bytes, nullptr, 8.f);
  if (st != ATTN_OK) return st;
  if (!dout || !dq || !dk || !dv || !delta) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      (reinterpret_cast<uintptr_t>(delta) & 3u))
    return ATTN_ERR_INVALID_ARG;
  const uint32_t flags = mask ? mask->flags : 0u;
  const int window = (flags & ATTN_WINDOW) ? mask->window : 0;
  const float cap = (flags & ATTN_SOFTCAP) ? mask->softcap : 0.f;
  const float* slopes = (mask && (flags & ATTN_ALIBI)) ? mask->alibi_slopes : nullptr;
  if (launch_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, H_kv, N, d, scale, flags, window, cap, slopes,
                 positional(mask) ? blockmap : nullptr, (hipStream_t)stream,
                 positional(mask) && compact_form(B, N, blockmap_bytes)) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status attn_bwd_gqa_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                 const void* dout, void* dq, void* dk, void* dv, int32_t B, int32_t H, int32_t H_kv,
                                 int32_t N, int32_t d, float scale, const attn_mask* mask, const void* blockmap,
                                 size_t blockmap_bytes, void* stream) {
  attn_status st = attn_check_args_gqa(q, k, v, const_cast<void*>(o), const_cast<float*>(lse), B, H, H_kv, N, d,
                                       scale, ATTN_BF16, mask, blockmap, blockmap_bytes, nullptr, 8.f);
  if (st != ATTN_OK) return st;
  if (!dout || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return ATTN_ERR_INVALID_ARG;
  if ((uint64_t)B * (uint64_t)H * (uint64_t)N > (uint64_t)bwd_scratch_rows()) return ATTN_ERR_INVALID_ARG;
  const uint32_t flags = mask ? mask->flags : 0u;
  const int window = (flags & ATTN_WINDOW) ? mask->window : 0;
  const float cap = (flags & ATTN_SOFTCAP) ? mask->softcap : 0.f;
  const float* slopes = (mask && (flags & ATTN_ALIBI)) ? mask->alibi_slopes : nullptr;
  if (launch_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, N, d, scale, flags, window, cap, slopes,
                         positional(mask) ? blockmap : nullptr, (hipStream_t)stream,
                         positional(mask) && compact_form(B, N, blockmap_bytes)) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                            const void* dout, void* dq, void* dk, void* dv, float* delta, int32_t H, int32_t H_kv,
                            int32_t total, int32_t d, float scale, const attn_mask* mask, const void* workspace,
                            size_t bytes, void* stream) {
  size_t need = 0;
  attn_status st = attn_varlen_workspace_bytes(total, mask, &need);
  if (st != ATTN_OK) return st;
  if (!workspace || !aligned16(workspace)) return ATTN_ERR_INVALID_ARG;
  if (bytes != need) return ATTN_ERR_BAD_BLOCKMAP;
  const attn_mask m = varlen_mask(mask, workspace, total);
  return attn_bwd_gqa(q, k, v, o, lse, dout, dq, dk, dv, delta, 1, H, H_kv, total, d, scale, &m, workspace,
                      varlen_doc_offset(total), stream);
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv, float* delta, int32_t B, int32_t H, int32_t N, int32_t d,
                     float scale, const attn_mask* mask, const void* blockmap, size_t blockmap_bytes,
                     void* stream) {
  return attn_bwd_gqa(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, H, N, d, scale, mask, blockmap,
                      blockmap_bytes, stream);
}

}  // extern "C"
