// FP8 block quantiser with incoherent processing (gfx950).
//
// "FlashAttention-3: Rekordverdächtige Geschwindigkeit und Präzision bei AI-Modellen"
// (ctol-digital.de), section "Analyse": FP8 keeps its accuracy through block
// quantisation and a processing step against outlier features (garbled on the page;
// read as FlashAttention-3's incoherent processing: Q and K multiplied by one random
// orthogonal matrix, R = D H / sqrt(d), random signs D and the Walsh-Hadamard matrix H,
// which leaves Q.K^T unchanged and spreads a large channel over all of them).
//
// One workgroup of 256 threads per (b*H + h, 128-row block), two rows per thread-quad
// pass (layout below):
//   widen bf16 -> fp32, flipping the signs on the way (an XOR of the bf16 sign bits);
//   with rotation run the fast Walsh-Hadamard transform, strides 1, 2, ..., d/2;
//   block maximum of |y| (wave shuffles, then LDS across the four waves);
//   s = amax / 448 and g = 448 / amax (both 1 for an all-zero block); the code is the
//   e4m3 value nearest to y / s, ties to even: y * g is within three fp32 ulps of y / s,
//   and where an e4m3 tie lies that close the sign of the exact residual y - t s (one
//   fma) moves it to the tie's correct side first (without rotation y is the input
//   itself, so the codes are those of the exact quotient); then v_cvt_pk_fp8_f32
//   (round to nearest even, subnormal codes kept, the sign of zero kept, nothing above
//   448 reachable since |y * g| <= 448 up to one rounding), written as 16-byte chunks;
//   the stored scale is s (times 1/sqrt(d) with rotation, so that code * scale
//   approximates x R; 1 for an all-zero block).
// HBM-bound: 2 bytes read and 1 written per element.
#include <algorithm>

#include "common.hpp"

namespace attn119 {

struct QuantArgs {
  const uint16_t* x;  // bf16 bits [BH][N][d]
  uint8_t* codes;     // [BH][N][d]
  float* scales;      // [BH][nblk]
  int N, nblk;
  int nwork;  // blocks in all: BH * nblk
  int rotate;
  float rnorm;            // fp32(1/sqrt(d))
  uint32_t sign_bits[4];  // element j negated when bit j%32 of word j/32 is set (zero
                          // without rotation)
};

// y * g (g = fp32(448 / amax), s = fp32(amax / 448)) as the value to round to e4m3, placed
// on the same side of every e4m3 tie as the exact quotient y / s: the product lies within
// three fp32 ulps of y / s, so only the midpoint t of the e4m3 interval holding it can lie
// between the two; when it is that close, the exact residual |y| - t s (one fma: its sign
// is exact) decides -- t itself when the quotient is the tie, else t moved one ulp towards
// the quotient.
__device__ __forceinline__ float e4m3_quotient(float y, float g, float s) {
  const float q = y * g;
  const float aq = __builtin_fabsf(q);
  // midpoint of the e4m3 interval of |q|: normal range (>= 2^-6): the exponent and top
  // three mantissa bits of |q| followed by a one; subnormal range: (k + 1/2) 2^-9
  const float t = aq >= 0x1p-6f ? __uint_as_float((__float_as_uint(aq) & 0xFFF00000u) | 0x80000u)
                                : ((float)(int)(aq * 512.f) + 0.5f) * 0x1p-9f;
  const int dist = (int)__float_as_uint(aq) - (int)__float_as_uint(t);
  if (dist > 4 || dist < -4) return q;
  const float r = __builtin_fmaf(-t, s, __builtin_fabsf(y));
  const float at = r == 0.f ? t : __uint_as_float(__float_as_uint(t) + (r > 0.f ? 1u : 0xFFFFFFFFu));
  return __builtin_copysignf(at, y);
}

// Whether e4m3_quotient may move q: in the normal range (|q| >= 2^-6) the midpoint of
// q's e4m3 interval has fp32 mantissa bits 19..0 equal to 0x80000, so q lies within four
// ulps of it exactly when those bits are in [0x7FFFC, 0x80004]; below 2^-6 (rare after the
// block scaling) every value counts as near.
__device__ __forceinline__ bool maybe_near_tie(float q) {
  const uint32_t b = __float_as_uint(q) & 0x7FFFFFFFu;
  return b < 0x3C800000u || ((b & 0xFFFFFu) - 0x7FFFCu) <= 8u;
}

// Lane layout: four lanes per row; lane k (0..3) of a row holds the 16-byte chunks
// q = 4c + k, c = 0 .. D/32 - 1, i.e. elements e = 8q + i.  Element bits 0-2 and 5-6 are
// in registers, bits 3-4 are the lane, so the transform strides 8 and 16 are quad
// permutations (DPP) and the others stay inside the thread; each load instruction of a
// wave reads 64 contiguous bytes of 16 rows.
template <int D>
__global__ void __launch_bounds__(256) quant_kernel(const QuantArgs a) {
  constexpr int NC = D / 32;  // chunks per lane per row
  const int wg = blockIdx.x;
  const int bh = wg / a.nblk, j = wg - bh * a.nblk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = tid & 3;
  const int r0 = j * 128 + (tid >> 2);  // rows r0 and r0 + 64

  // sign masks of this lane's pairs: pair (e, e+1), e = 8(4c + k) + 2m, sits in word c
  // of the sign bits at bit 8k + 2m
  uint32_t xm[NC][4];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t sw = a.sign_bits[c] >> (8 * k);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      xm[c][m] = (((sw >> (2 * m)) & 1u) << 15) | (((sw >> (2 * m + 1)) & 1u) << 31);
  }

  float v[2][NC][8];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = r0 + 64 * p;
    if (row < a.N) {
      const uint4* src = (const uint4*)(a.x + ((size_t)bh * a.N + row) * D);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint4 w = src[4 * c + k];
        const uint32_t ws[4] = {w.x ^ xm[c][0], w.y ^ xm[c][1], w.z ^ xm[c][2], w.w ^ xm[c][3]};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          v[p][c][2 * m] = __uint_as_float(ws[m] << 16);
          v[p][c][2 * m + 1] = __uint_as_float(ws[m] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[p][c][i] = 0.f;
    }
  }

  if (a.rotate) {
    // (x[e], x[e+h]) -> (x[e] + x[e+h], x[e] - x[e+h]) for h = 1, 2, 4, ..., D/2 in turn
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int h = 1; h < 8; h *= 2)
#pragma unroll
          for (int g = 0; g < 8; g += 2 * h)
#pragma unroll
            for (int i = g; i < g + h; ++i) {
              const float x0 = v[p][c][i], x1 = v[p][c][i + h];
              v[p][c][i] = x0 + x1;
              v[p][c][i + h] = x0 - x1;
            }
    // h = 8 and 16: the partner element sits in lane k ^ 1 (k ^ 2); the lane holding
    // x[e] forms o + v, the one holding x[e+h] forms o - v, both as one fma
    const float s8 = (k & 1) ? -1.f : 1.f, s16 = (k & 2) ? -1.f : 1.f;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float o = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[p][c][i]), 0xB1, 0xF, 0xF, false));
          v[p][c][i] = __builtin_fmaf(v[p][c][i], s8, o);
        }
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float o = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[p][c][i]), 0x4E, 0xF, 0xF, false));
          v[p][c][i] = __builtin_fmaf(v[p][c][i], s16, o);
        }
    // h = 32, 64 (D = 128: 32 only for D = 64): chunk slots c ^ 1, c ^ 2 of the thread
#pragma unroll
    for (int hc = 1; hc < NC; hc *= 2)
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          if ((c & hc) == 0)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float x0 = v[p][c][i], x1 = v[p][c + hc][i];
              v[p][c][i] = x0 + x1;
              v[p][c + hc][i] = x0 - x1;
            }
  }

  // block maximum of |y| (rows past N are zero)
  float mx = 0.f;
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[p][c][i]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
  __shared__ float s_max[4];
  if (lane == 0) s_max[wave] = mx;
  __syncthreads();
  const float amax = __builtin_fmaxf(__builtin_fmaxf(s_max[0], s_max[1]), __builtin_fmaxf(s_max[2], s_max[3]));
  // IEEE divisions (correctly rounded), once per block
  const float sc = amax > 0.f ? amax / 448.f : 1.f;
  const float g = amax > 0.f ? 448.f / amax : 1.f;

#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = r0 + 64 * p;
    if (row < a.N) {
      unsigned char* dst = a.codes + ((size_t)bh * a.N + row) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        // y * g, and the exact tie resolution only for the chunks of the wave where some
        // value lies near a tie (a wave-uniform branch: most chunks skip it)
        float w[8];
        bool near = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          w[i] = v[p][c][i] * g;
          near |= maybe_near_tie(w[i]);
        }
        if (__builtin_amdgcn_ballot_w64(near)) {
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i] = e4m3_quotient(v[p][c][i], g, sc);
        }
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(w[0], w[1], 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(w[2], w[3], lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(w[4], w[5], 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(w[6], w[7], hi, true);
        *(uint2*)(dst + 8 * (4 * c + k)) = make_uint2((uint32_t)lo, (uint32_t)hi);
      }
    }
  }
  if (tid == 0) a.scales[wg] = (a.rotate && amax > 0.f) ? sc * a.rnorm : sc;  // an all-zero block: 1
}

hipError_t launch_quant(const void* x, void* codes, float* scales, int BH, int N, int d, const uint32_t* signs,
                        hipStream_t stream) {
  QuantArgs a;
  a.x = (const uint16_t*)x;
  a.codes = (uint8_t*)codes;
  a.scales = scales;
  a.N = N;
  a.nblk = (N + 127) / 128;
  a.rotate = signs != nullptr;
  a.rnorm = (float)(1.0 / __builtin_sqrt((double)d));
  for (int i = 0; i < 4; ++i) a.sign_bits[i] = (signs && i < d / 32) ? signs[i] : 0u;
  a.nwork = BH * a.nblk;
  const dim3 grid((unsigned)a.nwork), block(256);
  if (d == 128) hipLaunchKernelGGL(quant_kernel<128>, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(quant_kernel<64>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn119
