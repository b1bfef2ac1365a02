// Shared device-side types and helpers for the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <utility>

namespace attn119 {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- direct HBM -> LDS loads the compiler does not track -----------------------------
// buffer_load ... lds writes each lane's data to LDS at M0 + W * lane.  Issued through the
// builtin, the compiler waits for such a load before any later LDS read it cannot prove
// disjoint from the destination (every read of a buffer chosen at run time), which makes
// a prefetch into one buffer wait before the first read of the other.  These helpers
// issue it where the compiler does not see it: the caller waits itself (s_waitcnt vmcnt,
// then a barrier) before anything reads the destination.  The instruction writes no
// register, so nothing the compiler allocates can be overwritten while it is in flight.
// The descriptor and the LDS address are wave-uniform (kept in SGPRs).  An SALU write of
// M0 needs one wait state before an LDS-DMA load reads it (the s_nop 0 between them; the
// compiler inserts it for its own loads, but not inside an asm statement).
// Descriptor of the bytes [base, base + bytes) (reads past the end give zero).
__device__ __forceinline__ u32x4 dma_rsrc(const void* base, int bytes) {
  const unsigned long long addr = (unsigned long long)base;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)addr),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(addr >> 32) & 0xFFFFu)),
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}
// W = 16: a 16-byte chunk per lane from descriptor offset voffset to LDS lds + 16 lane;
// W = 4: a dword per lane to lds + 4 lane.
template <int W>
__device__ __forceinline__ void dma_to_lds(u32x4 rs, __attribute__((address_space(3))) unsigned char* lds,
                                           int voffset) {
  static_assert(W == 16 || W == 4, "dword or 16-byte loads");
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(unsigned long long)lds);
  if constexpr (W == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voffset),
                 "s"(rs)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voffset),
                 "s"(rs)
                 : "memory", "m0");
}

// f(std::integral_constant<int, I>) for I = 0 .. N-1, unrolled by construction
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// v_permlane32_swap(a, b) exchanges the upper 32 lanes of a with the lower 32 lanes
// of b.  With a = b = x, lane l < 32 ends with (x[l], x[l+32]) and lane l >= 32 with
// (x[l-32], x[l]): both halves see the pair.  (The two results are copied out as
// integers before the bit casts: a bit cast applied to an element of the returned
// vector reads element 0 in this compiler.)
__device__ __forceinline__ void pair_of(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                                  false, false);
  const int r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
// max / sum of x over lanes l and l^32 (the two halves holding one query row)
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  pair_of(x, a, b);
  return __builtin_fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  pair_of(x, a, b);
  return a + b;
}

constexpr uint32_t kMapMagic = 0x39313141u;  // "A119"
constexpr int kBlock = 128;                  // block-map granularity (queries and keys)

// Work estimate of a query block in the work-order section of the map: a FULL key block
// is two 64-key steps, a PARTIAL one costs about 2.5 times as much (its mask code).
constexpr int kOrderFullCost = 2, kOrderPartialCost = 5;

constexpr uint32_t kCausal = 1, kWindow = 2, kDocument = 4, kAlibi = 8, kSoftcap = 16;
constexpr uint32_t kPositional = kCausal | kWindow | kDocument;

// Byte offsets of the block-map sections (see attn_blockmap_header in attn119.h).  The
// compact form (the workspace of a packed batch) has no class and list sections; their
// offsets are 0 there, and every other section is O(N).
struct MapLayout {
  size_t cls, counts, idx, row_lo, row_hi, col_lo, col_hi, pairs, status, order, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline MapLayout map_layout(int B, int N, bool compact = false) {
  const size_t nb = (size_t)((N + kBlock - 1) / kBlock);
  MapLayout m;
  size_t off = 256;  // header
  m.cls = compact ? 0 : off;
  if (!compact) off = align256(off + (size_t)B * nb * nb);
  m.counts = off;
  off = align256(off + (size_t)B * nb * 2 * 4);
  m.idx = compact ? 0 : off;
  if (!compact) off = align256(off + (size_t)B * nb * 2 * nb * 4);
  m.row_lo = off;
  off = align256(off + (size_t)B * N * 4);
  m.row_hi = off;
  off = align256(off + (size_t)B * N * 4);
  m.col_lo = off;
  off = align256(off + (size_t)B * N * 4);
  m.col_hi = off;
  off = align256(off + (size_t)B * N * 4);
  m.pairs = off;
  off = align256(off + (size_t)B * nb * 8);
  m.status = off;
  off = align256(off + (size_t)B * nb * 4);
  m.order = off;
  off = align256(off + (size_t)B * nb * 4);
  m.total = off;
  return m;
}

struct MapHeader {
  uint32_t magic;
  int32_t B, N, nqb, nkb;
  uint32_t flags;
  int32_t window;
  int32_t order_full_cost, order_partial_cost;  // weights of the work order (kOrder*Cost)
  int32_t compact;                              // 1: the compact form (no cls, no idx)
  int32_t reserved[6];
};

}  // namespace attn119
