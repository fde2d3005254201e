// Tile schedule built from cu_seqlens on the GPU.
//
// Every segment [c_s, c_{s+1}) is cut into tiles of `tile` rows counted from
// the segment's own start, so no tile straddles two documents.  A tile's work
// is the length of the key (or query) range it must visit:
//   prefix mode (forward, dQ): query tile t visits keys [0, min((t+1)*tile, L))
//   suffix mode (dK/dV):       key tile t visits queries [t*tile, L)
// Tiles outside a document's causal triangle are never listed ("Sample
// Packing：长序列 LLM 训练的 Attention 问题及优化", section 5.1: all-zero mask
// tiles need no work; the varlen decomposition turns the block-diagonal mask
// into one causal problem per document).
//
// Tiles are ordered by decreasing work (longest processing time first) with a
// counting sort over work measured in `unit`-row blocks.  Every stage is
// parallel over tiles: per-segment tile counts and their scan (one block), a
// histogram of tile bins, a descending scan of the bins, and a scatter in
// which each tile takes the next slot of its bin.  Ties are placed in atomic
// order; each tile's result does not depend on the order.
#include "psc_internal.h"

namespace psc {
namespace {

constexpr int kThreads = 256;

__device__ inline int32_t tile_work(int32_t L, int32_t t, int32_t tile, bool suffix) {
  return suffix ? L - t * tile : min((t + 1) * tile, L);
}

__device__ inline int32_t seg_len(const int32_t* cu, int32_t s, int32_t T) {
  const int32_t a = min(max(cu[s], 0), T);
  return min(max(cu[s + 1], a), T) - a;
}

// One block: zero the histogram, count each segment's tiles and scan them
// into toff[0..n_seg] (toff[n_seg] = number of tiles), and publish the count
// in n_items.  A count above the list's capacity (only a cu_seqlens that
// breaks its precondition gives one: clamped segments of a valid one hold at
// most T / tile + n_seg tiles) publishes 0 instead, because then some slots
// below the capacity could stay unwritten; with a count within capacity every
// slot below it is written (the slots of each bin, or each document's run,
// partition [0, count)).
__global__ void __launch_bounds__(kThreads) k_sched_tiles(const int32_t* cu, int32_t n_seg, int32_t T, int32_t tile,
                                                          int32_t* toff, int32_t* hist, int32_t n_bins,
                                                          int32_t* n_items, int64_t cap) {
  __shared__ int32_t wsum[kThreads / 64];
  for (int32_t i = threadIdx.x; i < n_bins; i += kThreads) hist[i] = 0;
  int32_t carry = 0;
  for (int32_t c = 0; c < n_seg; c += kThreads) {
    const int32_t s = c + threadIdx.x;
    int32_t v = 0;
    if (s < n_seg) v = (seg_len(cu, s, T) + tile - 1) / tile;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    int32_t off = 0, tot = 0;
    for (int k = 0; k < kThreads / 64; ++k) {
      if (k < wid) off += wsum[k];
      tot += wsum[k];
    }
    __syncthreads();
    if (s < n_seg) toff[s] = carry + off + x - v;
    carry += tot;
  }
  if (threadIdx.x == 0) {
    toff[n_seg] = carry;
    *n_items = (int64_t)carry <= cap ? carry : 0;
  }
}

// Tile i -> (segment, tile index inside it) by binary search over toff.
__device__ inline void tile_of(const int32_t* toff, int32_t n_seg, int32_t i, int32_t& s, int32_t& t) {
  int32_t lo = 0, hi = n_seg;  // toff[lo] <= i < toff[hi]
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (toff[mid] <= i) lo = mid; else hi = mid;
  }
  s = lo;
  t = i - toff[lo];
}

__device__ inline int32_t tile_bin(const int32_t* cu, int32_t s, int32_t t, int32_t T, int32_t tile, int32_t unit,
                                   bool suffix, int32_t n_bins) {
  const int32_t L = seg_len(cu, s, T);
  return min((tile_work(L, t, tile, suffix) + unit - 1) / unit, n_bins - 1);
}

__global__ void __launch_bounds__(kThreads) k_sched_count(const int32_t* cu, int32_t n_seg, int32_t T, int32_t tile,
                                                          int32_t unit, bool suffix, const int32_t* toff,
                                                          int32_t* hist, int32_t n_bins, int64_t cap) {
  const int32_t i = blockIdx.x * kThreads + threadIdx.x;
  const int32_t n = toff[n_seg];
  if (i >= n || i >= cap) return;
  int32_t s, t;
  tile_of(toff, n_seg, i, s, t);
  atomicAdd(&hist[tile_bin(cu, s, t, T, tile, unit, suffix, n_bins)], 1);
}

// Descending exclusive scan: cursor[b] = number of tiles in bins > b.
__global__ void __launch_bounds__(kThreads) k_sched_scan(int32_t* hist, int32_t n_bins) {
  __shared__ int32_t wsum[kThreads / 64];
  int32_t carry = 0;
  for (int32_t c = 0; c < n_bins; c += kThreads) {
    const int32_t i = c + threadIdx.x;
    const int32_t b = n_bins - 1 - i;  // walk bins from the top
    int32_t v = i < n_bins ? hist[b] : 0;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    int32_t off = 0, tot = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      if (w < wid) off += wsum[w];
      tot += wsum[w];
    }
    __syncthreads();
    if (i < n_bins) hist[b] = carry + off + x - v;
    carry += tot;
  }
}

__global__ void __launch_bounds__(kThreads) k_sched_fill(const int32_t* cu, int32_t n_seg, int32_t T, int32_t tile,
                                                         int32_t unit, bool suffix, const int32_t* toff,
                                                         int32_t* hist, int32_t n_bins, int32_t* items, int64_t cap) {
  const int32_t i = blockIdx.x * kThreads + threadIdx.x;
  const int32_t n = toff[n_seg];
  if (i >= n || i >= cap) return;
  int32_t s, t;
  tile_of(toff, n_seg, i, s, t);
  const int32_t pos = atomicAdd(&hist[tile_bin(cu, s, t, T, tile, unit, suffix, n_bins)], 1);
  if (pos < cap) {
    // the segment's clamped start and length travel with the item, so a
    // consumer needs one load (not item, then cu_seqlens) before its operands
    const int32_t a = min(max(cu[s], 0), T);
    *reinterpret_cast<int4*>(items + 4 * pos) = make_int4(a, seg_len(cu, s, T), t, s);
  }
}

// The whole schedule in one workgroup, for the common sizes (segments, bins
// and tiles few enough for LDS and one block's loops); one launch replaces
// four.  Prefix mode (forward, dQ) uses a document-major order: documents by
// decreasing length (counting sort over length bins), each taking a
// contiguous run of slots with its tiles by decreasing work (last tile
// first).  The query tiles of one document then run at the same time and
// read the same key/value prefix blocks together, which L2 serves once;
// this made the forward and dQ 10-13 % faster on 1-2K-token documents.  Suffix
// mode (dK/dV) keeps the plain longest-tile-first order, which measured
// faster there (workgroups of equal length run side by side, one per CU).
constexpr int kSmallThreads = 1024;
constexpr int kSmallSeg = 4096;     // n_seg + 1 limit (per-segment tables in LDS)
constexpr int kSmallBins = 4096;    // n_bins limit (histogram in LDS)
constexpr int64_t kSmallCap = 131072;

// Exclusive scan of v over the block (kSmallThreads lanes); returns this
// lane's prefix and the block total through `tot`.
__device__ inline int32_t block_exscan(int32_t v, int32_t* wsum, int32_t& tot) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  int32_t off = 0;
  tot = 0;
  for (int k = 0; k < kSmallThreads / 64; ++k) {
    if (k < wid) off += wsum[k];
    tot += wsum[k];
  }
  __syncthreads();
  return off + x - v;
}

__device__ inline int32_t doc_bin(const int32_t* cu, int32_t s, int32_t T, int32_t unit, int32_t n_bins) {
  return min((seg_len(cu, s, T) + unit - 1) / unit, n_bins - 1);
}

__global__ void __launch_bounds__(kSmallThreads) k_sched_small(const int32_t* cu, int32_t n_seg, int32_t T,
                                                               int32_t tile, int32_t unit, bool suffix,
                                                               int32_t n_bins, int32_t* items, int64_t cap,
                                                               int32_t* n_items) {
  __shared__ int32_t toff[kSmallSeg];
  __shared__ int32_t dpos[kSmallSeg];  // prefix mode: first slot of each document's run
  __shared__ int32_t hist[kSmallBins];
  __shared__ int32_t wsum[kSmallThreads / 64];
  for (int32_t i = threadIdx.x; i < n_bins; i += kSmallThreads) hist[i] = 0;
  // tiles per segment, scanned into toff[0..n_seg]
  int32_t carry = 0;
  for (int32_t c = 0; c < n_seg; c += kSmallThreads) {
    const int32_t sg = c + threadIdx.x;
    const int32_t v = sg < n_seg ? (seg_len(cu, sg, T) + tile - 1) / tile : 0;
    int32_t tot;
    const int32_t ex = block_exscan(v, wsum, tot);
    if (sg < n_seg) toff[sg] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) toff[n_seg] = carry;
  __syncthreads();
  // beyond the capacity (a cu_seqlens that breaks its precondition) nothing
  // is listed: part of the slots could otherwise stay unwritten
  const int32_t n = (int64_t)carry <= cap ? carry : 0;
  if (suffix) {
    // longest tile first: histogram of tile work
    for (int32_t i = threadIdx.x; i < n; i += kSmallThreads) {
      int32_t sg, t;
      tile_of(toff, n_seg, i, sg, t);
      atomicAdd(&hist[tile_bin(cu, sg, t, T, tile, unit, true, n_bins)], 1);
    }
  } else {
    // document-major: tiles per document-length bin
    for (int32_t sg = threadIdx.x; sg < n_seg; sg += kSmallThreads)
      atomicAdd(&hist[doc_bin(cu, sg, T, unit, n_bins)], toff[sg + 1] - toff[sg]);
  }
  __syncthreads();
  // descending exclusive scan: cursor[b] = tiles of the documents in bins above b
  carry = 0;
  for (int32_t c = 0; c < n_bins; c += kSmallThreads) {
    const int32_t i = c + threadIdx.x;
    const int32_t b = n_bins - 1 - i;
    const int32_t v = i < n_bins ? hist[b] : 0;
    int32_t tot;
    const int32_t ex = block_exscan(v, wsum, tot);
    if (i < n_bins) hist[b] = carry + ex;
    carry += tot;
  }
  __syncthreads();
  if (!suffix) {
    // each document claims a contiguous run inside its bin
    for (int32_t sg = threadIdx.x; sg < n_seg; sg += kSmallThreads)
      dpos[sg] = atomicAdd(&hist[doc_bin(cu, sg, T, unit, n_bins)], toff[sg + 1] - toff[sg]);
    __syncthreads();
  }
  // scatter: suffix mode takes the next slot of the tile's work bin; prefix
  // mode puts tile t of document sg at its run's slot nt - 1 - t
  for (int32_t i = threadIdx.x; i < n; i += kSmallThreads) {
    int32_t sg, t;
    tile_of(toff, n_seg, i, sg, t);
    const int32_t pos = suffix ? atomicAdd(&hist[tile_bin(cu, sg, t, T, tile, unit, true, n_bins)], 1)
                               : dpos[sg] + (toff[sg + 1] - toff[sg]) - 1 - t;
    if (pos < n) {
      const int32_t a = min(max(cu[sg], 0), T);
      *reinterpret_cast<int4*>(items + 4 * pos) = make_int4(a, seg_len(cu, sg, T), t, sg);
    }
  }
  if (threadIdx.x == 0) *n_items = n;
}

}  // namespace

// Upper bound on the number of tiles: sum over segments of ceil(L / tile)
// <= T / tile + n_seg.
static int64_t sched_cap(int64_t T, int32_t n_seg, int tile) { return T / tile + n_seg + 1; }
static int32_t sched_bins(int32_t max_seqlen, int unit) { return (max_seqlen + unit - 1) / unit + 2; }

size_t schedule_bytes(int64_t T, int32_t n_seg, int32_t max_seqlen, int tile, int unit) {
  return align_up(sizeof(int32_t) * 4 * sched_cap(T, n_seg, tile), 256) +
         align_up(sizeof(int32_t) * sched_bins(max_seqlen, unit), 256) +
         align_up(sizeof(int32_t) * ((size_t)n_seg + 1), 256) + 256;
}

TileSchedule schedule_carve(void* ws, int64_t T, int32_t n_seg, int32_t max_seqlen, int tile, int unit) {
  TileSchedule s;
  char* p = static_cast<char*>(ws);
  s.cap = sched_cap(T, n_seg, tile);
  s.n_bins = sched_bins(max_seqlen, unit);
  s.items = reinterpret_cast<int32_t*>(p);
  p += align_up(sizeof(int32_t) * 4 * s.cap, 256);
  s.hist = reinterpret_cast<int32_t*>(p);
  p += align_up(sizeof(int32_t) * s.n_bins, 256);
  s.toff = reinterpret_cast<int32_t*>(p);
  p += align_up(sizeof(int32_t) * ((size_t)n_seg + 1), 256);
  s.n_items = reinterpret_cast<int32_t*>(p);
  return s;
}

hipError_t launch_schedule(const int32_t* cu, int32_t n_seg, int32_t T, int tile, int unit, bool suffix,
                           const TileSchedule& s, hipStream_t stream) {
  ScopedKernelTimer timed(kTimeSchedule, stream);
  if (n_seg + 1 <= kSmallSeg && s.n_bins <= kSmallBins && s.cap <= kSmallCap) {
    k_sched_small<<<1, kSmallThreads, 0, stream>>>(cu, n_seg, T, tile, unit, suffix, s.n_bins, s.items, s.cap,
                                                   s.n_items);
    return hipGetLastError();
  }
  const unsigned gt = (unsigned)((s.cap + kThreads - 1) / kThreads);
  k_sched_tiles<<<1, kThreads, 0, stream>>>(cu, n_seg, T, tile, s.toff, s.hist, s.n_bins, s.n_items, s.cap);
  k_sched_count<<<gt, kThreads, 0, stream>>>(cu, n_seg, T, tile, unit, suffix, s.toff, s.hist, s.n_bins, s.cap);
  k_sched_scan<<<1, kThreads, 0, stream>>>(s.hist, s.n_bins);
  k_sched_fill<<<gt, kThreads, 0, stream>>>(cu, n_seg, T, tile, unit, suffix, s.toff, s.hist, s.n_bins, s.items,
                                            s.cap);
  return hipGetLastError();
}

}  // namespace psc
