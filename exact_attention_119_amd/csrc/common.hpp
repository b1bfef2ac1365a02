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

// f(std::integral_constant<int, I>) for I = 0 .. N-1, unrolled by construction
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr uint32_t kMapMagic = 0x39313141u;  // "A119"
constexpr int kBlock = 128;                  // block-map granularity (queries and keys)

// Work estimate of a query block in the work-order section of the map: a FULL key block
// is two 64-key steps, a PARTIAL one costs about 2.5 times as much (its mask code).
constexpr int kOrderFullCost = 2, kOrderPartialCost = 5;

constexpr uint32_t kCausal = 1, kWindow = 2, kDocument = 4, kAlibi = 8, kSoftcap = 16;
constexpr uint32_t kPositional = kCausal | kWindow | kDocument;

// Byte offsets of the block-map sections (see attn_blockmap_header in attn119.h).
struct MapLayout {
  size_t cls, counts, idx, row_lo, row_hi, pairs, status, order, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline MapLayout map_layout(int B, int N) {
  const size_t nb = (size_t)((N + kBlock - 1) / kBlock);
  MapLayout m;
  size_t off = 256;  // header
  m.cls = off;
  off = align256(off + (size_t)B * nb * nb);
  m.counts = off;
  off = align256(off + (size_t)B * nb * 2 * 4);
  m.idx = off;
  off = align256(off + (size_t)B * nb * 2 * nb * 4);
  m.row_lo = off;
  off = align256(off + (size_t)B * N * 4);
  m.row_hi = off;
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
  int32_t reserved[7];
};

}  // namespace attn119
