// Block-map builder for the fused attention forward pass (gfx950).
//
// Block sparsity -- skipping blocks the mask hides completely -- is named in
// "PyTorchs FlexAttention mit FlashAttention-4 ist ein Game-Changer" (liora.io),
// section "Aktuelle Einschränkungen".  Every mask this library supports (causal,
// sliding window, document with contiguous documents, and their conjunctions)
// leaves each query row a single interval of visible keys [row_lo, row_hi], so
// the map is built from those intervals, in one launch with one workgroup per
// 128-row query block:
//   its rows (one thread each): the interval of keys the row sees and the interval of
//          rows that see the row's position as a key, and a flag for any place where doc_id
//          decreases (documents must be contiguous runs), giving the block's status
//          word: 1 if doc_id decreases at one of its rows, or, for a packed batch, if
//          its share of the sequence offsets is out of order (a batch row with any
//          such word is invalid);
//   its row of blocks: the class of every 128x128 block, the ascending lists of FULL
//          and PARTIAL key blocks and the visible-pair count of the query block.
// The compact form (the workspace of a packed batch, read only by the forward pass) has
// no class and list sections, so that it grows as O(N): its FULL and PARTIAL counts come
// from the intervals of the block's first and last rows r0 and r1 alone.  Every row sees
// itself and both ends of the intervals are non-decreasing in the row, so the rows'
// intervals together cover [lo(r0), hi(r1)] without a gap (the non-empty key blocks are
// those that meet it), and a key block is FULL exactly when it lies inside
// [lo(r1), hi(r0)] with 128 keys and the query block has 128 rows.
// For a packed batch the rows' sequences come from the offsets, and the kernel also
// writes the sequence id of every token to the workspace.
// A second launch, for document masks only, fills the work-order section: the
// (batch row, query block) pairs heaviest-first by the work of their block lists (other
// masks keep the identity order the first launch writes; their work is known from the
// row index).
// No atomics, no memset: every byte of every section is written, so the result is
// byte-identical for equal inputs and the calls are safe to capture in a graph.
#include "common.hpp"

namespace attn119 {

struct MapArgs {
  unsigned char* map;
  MapLayout lay;
  const int32_t* doc_id;
  int B, N, nb;
  uint32_t flags;  // positional flags only
  int window;
  const int32_t* cu;  // packed variable-length batch (B = 1): offsets [nseq + 1], else null
  int nseq;
  int32_t* ids;       // packed batch: the sequence id of every token, written here
  int compact;        // 1: the compact form (no class and list sections)
};

// Narrows a search interval [lo, hi] after a round whose probes lo + t*step (t < 256)
// found the predicate true at c of them (a prefix when the row is sorted).
__device__ inline void narrow(int& lo, int& hi, int step, int c, bool& done) {
  if (c == 0) { done = true; return; }  // false already at lo
  const int base = lo;
  lo = base + (c - 1) * step + 1;
  hi = min(base + c * step, hi);
  done = lo >= hi;
}

// Two searches over one non-decreasing row, by the whole workgroup: lower = first index
// with row[i] >= va, upper = first index with row[i] > vb (both in [0, N]).  Each round
// the 256 threads probe evenly spaced positions of both intervals left and keep the gap
// where the predicate turns false, so N <= 65536 takes two rounds of loads; the first
// round's probes sit at fixed positions and come in with the caller's other loads
// (pv0 = row[tid * ceil(N/256)] where that is < N).  Must be reached by all threads with
// the same arguments; for any row contents both results stay in [0, N] and the loop ends
// (each interval shrinks to below 1/256 per round).
__device__ void par_bounds(const int32_t* row, int N, int pv0, int va, int vb, int& lower, int& upper) {
  const int t = threadIdx.x;
  int lo_a = 0, hi_a = N, lo_b = 0, hi_b = N;
  bool da = false, db = false;
  {
    const int step = (N + 255) / 256;
    const bool in = t * step < N;
    const int ca = __syncthreads_count(in && pv0 < va);
    const int cb = __syncthreads_count(in && pv0 <= vb);
    narrow(lo_a, hi_a, step, ca, da);
    narrow(lo_b, hi_b, step, cb, db);
  }
  while (!da || !db) {
    const int sa = (hi_a - lo_a + 255) / 256, sb = (hi_b - lo_b + 255) / 256;
    const int pa = lo_a + t * sa, pb = lo_b + t * sb;
    const bool ia = !da && pa < hi_a, ib = !db && pb < hi_b;
    const int xa = ia ? row[pa] : 0, xb = ib ? row[pb] : 0;
    const int ca = __syncthreads_count(ia && xa < va);
    const int cb = __syncthreads_count(ib && xb <= vb);
    if (!da) narrow(lo_a, hi_a, sa, ca, da);
    if (!db) narrow(lo_b, hi_b, sb, cb, db);
  }
  lower = lo_a;
  upper = lo_b;
}

// One workgroup (256 threads, 4 waves) per (query block, batch row): the intervals and
// the status word of its 128 rows, then the classes and lists of its row of blocks.
__global__ void __launch_bounds__(256) blockmap_kernel(MapArgs a) {
  const int qb = blockIdx.x, b = blockIdx.y;
  const int N = a.N, nb = a.nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q0 = qb * kBlock, q1 = min(N, q0 + kBlock);
  const int nrows = q1 - q0;

  __shared__ int s_lo[kBlock], s_hi[kBlock];
  __shared__ int s_wave_full[4], s_wave_part[4];
  __shared__ long long s_pairs[4];

  // ---- row intervals (threads 0..127, one query row each) and the status word ----------
  // Documents: the rows' ids (and the next row's) go to LDS; a row's document starts at
  // the first row of its run in the block, or, for the run that reaches the block's first
  // row, where that document starts in the batch row (one search for the workgroup), and
  // ends likewise.
  __shared__ int s_doc[kBlock + 1];
  __shared__ int s_run_f[4], s_run_g[4];
  int first0 = 0, last1 = N - 1, run_first = 0, run_last = 0;
  // Packed batches: a row's sequence is the number of interior offsets cu[1..nseq-1] at
  // or below it (a binary search; every read stays inside cu whatever the values), its
  // bounds cu[id] and cu[id + 1] - 1; the ids go to the workspace from here.  Offsets out
  // of order give wrong bounds, and the check below marks the batch row invalid.
  int cu_ds = 0, cu_de = N - 1;
  if (a.cu) {
    if (tid < nrows) {
      const int q = q0 + tid;
      int lo = 1, hi = a.nseq;  // first index in [1, nseq) with cu[index] > q
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a.cu[mid] <= q) lo = mid + 1; else hi = mid;
      }
      const int sq = lo - 1;
      a.ids[q] = sq;
      cu_ds = a.cu[sq];
      cu_de = a.cu[sq + 1] - 1;
    }
  } else if (a.flags & kDocument) {
    const int32_t* drow = a.doc_id + (size_t)b * N;
    const int step0 = (N + 255) / 256;
    const int pv0 = tid * step0 < N ? drow[tid * step0] : 0;
    if (tid <= nrows && q0 + tid < N) s_doc[tid] = drow[q0 + tid];
    __syncthreads();
    int past1;
    par_bounds(drow, N, pv0, s_doc[0], s_doc[nrows - 1], first0, past1);
    last1 = past1 - 1;
    // runs of equal ids inside the block: the first row of this row's run is the
    // largest run start at or before it (prefix max over the rows), the last row the
    // smallest run end at or after it (suffix min); threads 0..127 are waves 0 and 1
    int f = tid, g = tid;  // rows past the block's end count as runs of their own
    if (tid < nrows) {
      const int dq = s_doc[tid];
      f = (tid == 0 || s_doc[tid - 1] != dq) ? tid : -1;
      g = (tid == nrows - 1 || s_doc[tid + 1] != dq) ? tid : INT32_MAX;
    }
    for (int off = 1; off < 64; off <<= 1) {
      const int fu = __shfl_up(f, off), gd = __shfl_down(g, off);
      if (lane >= off) f = max(f, fu);
      if (lane + off < 64) g = min(g, gd);
    }
    if (lane == 63) s_run_f[wave] = f;
    if (lane == 0) s_run_g[wave] = g;
    __syncthreads();
    run_first = wave == 1 ? max(f, s_run_f[0]) : f;
    run_last = wave == 0 ? min(g, s_run_g[1]) : g;
  }
  int bad = 0;
  if (tid < kBlock) {
    int lo = 0, hi = -1;
    if (tid < nrows) {
      const int q = q0 + tid;
      lo = 0;
      hi = N - 1;
      if (a.flags & kCausal) hi = q;
      if (a.flags & kWindow) {
        lo = max(lo, q - (a.window - 1));
        if (!(a.flags & kCausal)) hi = min(hi, q + (a.window - 1));
      }
      // the rows that see key q (position q as a key): the same predicates with the
      // roles swapped
      int clo = (a.flags & kCausal) ? q : 0, chi = N - 1;
      if (a.flags & kWindow) {
        if (!(a.flags & kCausal)) clo = max(0, q - (a.window - 1));
        chi = min(chi, q + (a.window - 1));
      }
      if (a.flags & kDocument) {
        int ds = cu_ds, de = cu_de;
        if (!a.cu) {
          if (q + 1 < N && s_doc[tid + 1] < s_doc[tid]) bad = 1;
          ds = run_first == 0 ? first0 : q0 + run_first;
          de = run_last == nrows - 1 ? last1 : q0 + run_last;
        }
        lo = max(lo, ds);
        hi = min(hi, de);
        clo = max(clo, ds);
        chi = min(chi, de);
      }
      if (hi < lo) { lo = 0; hi = -1; }
      if (chi < clo) { clo = 0; chi = -1; }
      ((int32_t*)(a.map + a.lay.row_lo))[(size_t)b * N + q] = lo;
      ((int32_t*)(a.map + a.lay.row_hi))[(size_t)b * N + q] = hi;
      ((int32_t*)(a.map + a.lay.col_lo))[(size_t)b * N + q] = clo;
      ((int32_t*)(a.map + a.lay.col_hi))[(size_t)b * N + q] = chi;
    }
    s_lo[tid] = lo;
    s_hi[tid] = hi;
  }
  // Packed batches: the doc ids came from cu by binary search, which is exact only for
  // offsets that run from 0 to N without decreasing.  The workgroups share the check of
  // that: workgroup qb takes the pairs (cu[i], cu[i+1]) with i = qb*256 + tid + k*nb*256.
  if (a.cu) {
    for (int i = qb * 256 + tid; i < a.nseq; i += nb * 256)
      if (a.cu[i] > a.cu[i + 1]) bad = 1;
    if (qb == 0 && tid == 0 && (a.cu[0] != 0 || a.cu[a.nseq] != N)) bad = 1;
  }
  // status: 1 if doc_id decreases between one of this block's rows and the next row (or
  // the offsets this workgroup checked are out of order)
  const int bad_any = __syncthreads_or(bad);  // (also orders the interval writes above)
  if (tid == 0) ((int32_t*)(a.map + a.lay.status))[(size_t)b * nb + qb] = bad_any ? 1 : 0;

  // visible pairs of this query block
  long long my_pairs = 0;
  if (tid < kBlock) my_pairs = (long long)max(0, s_hi[tid] - s_lo[tid] + 1);
  for (int off = 32; off > 0; off >>= 1) my_pairs += __shfl_xor(my_pairs, off);
  if (lane == 0) s_pairs[wave] = my_pairs;
  __syncthreads();

  int full_base = 0, part_base = 0;
  if (a.compact) {
    // counts from the first and last rows' intervals (an empty row, possible only in a
    // batch row marked invalid, has [0, -1])
    const int lo0 = s_lo[0], lo1 = s_lo[nrows - 1], hi0 = s_hi[0], hi1 = s_hi[nrows - 1];
    const int ua = lo0 / kBlock, ub = hi1 < 0 ? -1 : hi1 / kBlock;
    const int nne = max(0, ub - ua + 1);
    const int fa = (lo1 + kBlock - 1) / kBlock, fz = (hi0 + 1) / kBlock - 1;
    full_base = nrows == kBlock ? min(max(0, fz - fa + 1), nne) : 0;
    part_base = nne - full_base;
  } else {
    unsigned char* cls = a.map + a.lay.cls + ((size_t)b * nb + qb) * nb;
    int32_t* idx_full = (int32_t*)(a.map + a.lay.idx) + ((size_t)b * nb + qb) * 2 * nb;
    int32_t* idx_part = idx_full + nb;

    // classes and ascending CSR lists, up to 256 key blocks per round.  Wave w holds rows
    // 64*(w%2) + lane (their intervals in registers) and tests the key blocks of parity w/2
    // against all of them at once: one ballot for "some row sees a key of the block", one
    // for "every row sees all of it".
    __shared__ unsigned char s_any[2][256], s_all[2][256];
    const int half = wave & 1;
    const int my_lo = s_lo[64 * half + lane], my_hi = s_hi[64 * half + lane];
    for (int kb0 = 0; kb0 < nb; kb0 += 256) {
      const int K = min(256, nb - kb0);
      for (int kl = wave >> 1; kl < K; kl += 2) {
        const int k0 = (kb0 + kl) * kBlock, k1 = min(N, k0 + kBlock) - 1;
        const uint64_t any = __ballot(max(my_lo, k0) <= min(my_hi, k1));
        const uint64_t all = __ballot(my_lo <= k0 && my_hi >= k1);
        if (lane == 0) {
          s_any[half][kl] = any != 0;
          s_all[half][kl] = all == ~0ull;
        }
      }
      __syncthreads();
      const int kb = kb0 + tid;
      int c = 0;
      if (tid < K) {
        const int k0 = kb * kBlock, k1 = min(N, k0 + kBlock) - 1;
        const bool any = s_any[0][tid] | s_any[1][tid];
        const bool all = s_all[0][tid] & s_all[1][tid] & (nrows == kBlock) & (k1 - k0 + 1 == kBlock);
        c = !any ? 0 : (all ? 2 : 1);
        cls[kb] = (unsigned char)c;
      }
      const uint64_t mfull = __ballot(c == 2);
      const uint64_t mpart = __ballot(c == 1);
      if (lane == 0) {
        s_wave_full[wave] = __popcll(mfull);
        s_wave_part[wave] = __popcll(mpart);
      }
      __syncthreads();
      int fb = full_base, pbase = part_base;
      for (int w = 0; w < wave; ++w) { fb += s_wave_full[w]; pbase += s_wave_part[w]; }
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      if (c == 2) idx_full[fb + __popcll(mfull & below)] = kb;
      if (c == 1) idx_part[pbase + __popcll(mpart & below)] = kb;
      for (int w = 0; w < 4; ++w) { full_base += s_wave_full[w]; part_base += s_wave_part[w]; }
      __syncthreads();
    }
    for (int i = full_base + tid; i < nb; i += 256) idx_full[i] = -1;
    for (int i = part_base + tid; i < nb; i += 256) idx_part[i] = -1;
  }
  if (tid == 0 && b == 0 && qb == 0) {
    MapHeader* hd = (MapHeader*)a.map;
    hd->magic = kMapMagic;
    hd->B = a.B;
    hd->N = a.N;
    hd->nqb = nb;
    hd->nkb = nb;
    hd->flags = a.flags;
    hd->window = a.window;
    hd->order_full_cost = kOrderFullCost;
    hd->order_partial_cost = kOrderPartialCost;
    hd->compact = a.compact;
    for (int i = 0; i < 6; ++i) hd->reserved[i] = 0;
  }
  if (tid == 0) {
    int32_t* counts = (int32_t*)(a.map + a.lay.counts) + ((size_t)b * nb + qb) * 2;
    counts[0] = full_base;
    counts[1] = part_base;
    long long* pairs = (long long*)(a.map + a.lay.pairs) + (size_t)b * nb + qb;
    *pairs = s_pairs[0] + s_pairs[1] + s_pairs[2] + s_pairs[3];
    ((int32_t*)(a.map + a.lay.order))[(size_t)b * nb + qb] = b * nb + qb;  // identity order
  }
}

// Work order for document masks: entry e = b * nb + qb has the work estimate
// w(e) = kOrderFullCost * #FULL + kOrderPartialCost * #PARTIAL, and goes to position
// rank(e) = #{e' : w(e') > w(e), or w(e') == w(e) and e' < e} -- a permutation of
// 0 .. M-1 (heaviest first, ties in index order).  One thread per entry; every
// workgroup streams all M estimates through LDS in chunks.
__global__ void __launch_bounds__(256) order_kernel(const int32_t* counts, int32_t* order, int M) {
  constexpr int CH = 1024;
  __shared__ int s_w[CH];
  const int e = blockIdx.x * 256 + threadIdx.x;
  auto work = [&](int i) { return kOrderFullCost * counts[2 * i] + kOrderPartialCost * counts[2 * i + 1]; };
  const int we = e < M ? work(e) : 0;
  int rank = 0;
  for (int c0 = 0; c0 < M; c0 += CH) {
    const int n = min(CH, M - c0);
    for (int i = threadIdx.x; i < n; i += 256) s_w[i] = work(c0 + i);
    __syncthreads();
    for (int i = 0; i < n; ++i) {
      const int w = s_w[i];
      rank += (w > we) | ((w == we) & (c0 + i < e));
    }
    __syncthreads();
  }
  if (e < M) order[rank] = e;
}

hipError_t launch_blockmap(unsigned char* map, int B, int N, uint32_t flags, int window,
                           const int32_t* doc_id, const int32_t* cu, int nseq, int32_t* ids, bool compact,
                           hipStream_t stream) {
  MapArgs a;
  a.map = map;
  a.lay = map_layout(B, N, compact);
  a.compact = compact ? 1 : 0;
  a.doc_id = doc_id;
  a.B = B;
  a.N = N;
  a.nb = (N + kBlock - 1) / kBlock;
  a.flags = flags & kPositional;
  a.window = window;
  a.cu = cu;
  a.nseq = nseq;
  a.ids = ids;
  hipLaunchKernelGGL(blockmap_kernel, dim3(a.nb, B), dim3(256), 0, stream, a);
  if (a.flags & kDocument) {
    const int M = B * a.nb;
    hipLaunchKernelGGL(order_kernel, dim3((M + 255) / 256), dim3(256), 0, stream,
                       (const int32_t*)(map + a.lay.counts), (int32_t*)(map + a.lay.order), M);
  }
  return hipGetLastError();
}

}  // namespace attn119
