// Sample packing on the GPU: build_pack (carry-over) and build_unpack
// (truncate to SEQ_LEN, at most micro_bsz documents a row, zero pad).
//
// Rules: InternEvo documentation, "数据加载与流程", section "Dataloader加载数据"
// (both packers and the label rule) and section "获取Dataloader数据"
// (cu_seqlens: every row starts a segment, every document start inside a row
// starts one, the padding tail is a segment; indexes count from 0 in each).
//
// Pipeline (all integer work, bound by launch latency at the sizes used here
// and by HBM bandwidth beyond):
//   1. scan over documents (reduce-then-scan, three kernels): for every
//      document the number of non-empty documents before it and the sum of
//      their truncated lengths; plus the list of non-empty documents.
//   2. per row: valid length, segment count and a base offset.
//   3. scan over rows of the segment counts -> row_seg_ptr; statistics.
//   4. emit: input_ids, labels, indexes for every output position.
//   5. boundaries: each row start, document start and padding start writes its
//      own cu_seqlens entry (the slot is known from the scans, no sorting).
//   6. longest segment: max reduction of adjacent cu_seqlens differences.
#include "psc_internal.h"

namespace psc {
namespace {

constexpr int kThreads = 256;
constexpr int kItems = kScanTile / kThreads;  // 4 documents per thread
static_assert(kItems * kThreads == kScanTile, "scan tile");

struct Pair {
  long long a, b;
};
__device__ inline Pair operator+(Pair x, Pair y) { return {x.a + y.a, x.b + y.b}; }
__device__ inline Pair operator-(Pair x, Pair y) { return {x.a - y.a, x.b - y.b}; }

// Value scanned for document d (d == n_docs contributes nothing): whether it is
// non-empty, and its length cut to seq_len.
__device__ inline Pair doc_value(const int64_t* off, int64_t n_docs, int64_t n_tokens, int32_t seq_len,
                                 int64_t d) {
  if (d >= n_docs) return {0, 0};
  int64_t s = min(max(off[d], (int64_t)0), n_tokens);
  int64_t e = min(max(off[d + 1], s), n_tokens);
  int64_t len = e - s;
  return {len > 0 ? 1 : 0, len > 0 ? (long long)min(len, (int64_t)seq_len) : 0};
}

// Inclusive scan across a 64-lane wave, then across the block's waves.
// Returns the exclusive prefix of `v`; *total receives the block total.
__device__ inline Pair block_exclusive_scan(Pair v, Pair* total, Pair* lds) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  Pair x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    long long ya = __shfl_up(x.a, o, 64), yb = __shfl_up(x.b, o, 64);
    if (lane >= o) {
      x.a += ya;
      x.b += yb;
    }
  }
  if (lane == 63) lds[wid] = x;
  __syncthreads();
  Pair off = {0, 0}, tot = {0, 0};
  for (int w = 0; w < kThreads / 64; ++w) {
    if (w < wid) off = off + lds[w];
    tot = tot + lds[w];
  }
  __syncthreads();
  *total = tot;
  return x - v + off;
}

__global__ void __launch_bounds__(kThreads) k_scan_partial(const int64_t* off, int64_t n_docs, int64_t n_tokens,
                                                            int32_t seq_len, int64_t* partials) {
  __shared__ Pair lds[kThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kItems;
  Pair s = {0, 0};
  for (int i = 0; i < kItems; ++i) s = s + doc_value(off, n_docs, n_tokens, seq_len, base + i);
  Pair tot;
  block_exclusive_scan(s, &tot, lds);
  if (threadIdx.x == 0) {
    partials[2 * blockIdx.x] = tot.a;
    partials[2 * blockIdx.x + 1] = tot.b;
  }
}

// One block turns the per-block totals into exclusive block offsets.
__global__ void __launch_bounds__(kThreads) k_scan_top(int64_t* partials, int64_t n_blocks) {
  __shared__ Pair lds[kThreads / 64];
  Pair carry = {0, 0};
  for (int64_t c = 0; c < n_blocks; c += kThreads) {
    int64_t i = c + threadIdx.x;
    Pair v = i < n_blocks ? Pair{partials[2 * i], partials[2 * i + 1]} : Pair{0, 0};
    Pair tot;
    Pair ex = block_exclusive_scan(v, &tot, lds);
    if (i < n_blocks) {
      partials[2 * i] = carry.a + ex.a;
      partials[2 * i + 1] = carry.b + ex.b;
    }
    carry = carry + tot;
  }
}

__global__ void __launch_bounds__(kThreads) k_scan_final(const int64_t* off, int64_t n_docs, int64_t n_tokens,
                                                          int32_t seq_len, const int64_t* partials,
                                                          int64_t* nz_rank, int64_t* trunc_scan,
                                                          int64_t* slot_doc) {
  __shared__ Pair lds[kThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kItems;
  Pair v[kItems];
  Pair s = {0, 0};
  for (int i = 0; i < kItems; ++i) {
    v[i] = doc_value(off, n_docs, n_tokens, seq_len, base + i);
    s = s + v[i];
  }
  Pair tot;
  Pair run = block_exclusive_scan(s, &tot, lds);
  run = run + Pair{partials[2 * blockIdx.x], partials[2 * blockIdx.x + 1]};
  for (int i = 0; i < kItems; ++i) {
    int64_t d = base + i;
    if (d <= n_docs) {
      nz_rank[d] = run.a;
      trunc_scan[d] = run.b;
      if (v[i].a) slot_doc[run.a] = d;
    }
    run = run + v[i];
  }
}

// First index i in [0, n] with a[i] > x (a non-decreasing).
__device__ inline int64_t upper_bound(const int64_t* a, int64_t n, int64_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}
// First index i in [0, n] with a[i] >= x.
__device__ inline int64_t lower_bound(const int64_t* a, int64_t n, int64_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ inline int64_t clamp_off(const int64_t* off, int64_t d, int64_t n_tokens) {
  return min(max(off[d], (int64_t)0), n_tokens);
}

struct RowCtx {
  int mode;
  const int64_t* off;
  int64_t n_docs, n_tokens, n_rows;
  int32_t mb, seq_len, PL;
  const int64_t *nz_rank, *trunc_scan, *slot_doc;
  int64_t* row_aux;
  int32_t* row_valid;
  int32_t* row_cnt;      // row_seg_ptr used as per-row counts before the row scan
  int32_t* valid_out;    // optional user output
};

// Per row: valid length, number of segments, and a base used later.
//   carry-over: base = number of non-empty documents starting at or before the
//               row start (so a document's rank inside the row follows);
//   truncate:   base = truncated-stream offset of the row's first document.
__global__ void __launch_bounds__(kThreads) k_row_count(RowCtx c) {
  int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (r >= c.n_rows) return;
  const int64_t row0 = r * c.PL;
  int32_t valid, segs;
  int64_t aux;
  if (c.mode == 0) {
    valid = (int32_t)min((int64_t)c.PL, c.n_tokens - row0);
    int64_t lo = upper_bound(c.off, c.n_docs + 1, row0);           // first start > row0
    int64_t hi = lower_bound(c.off, c.n_docs + 1, row0 + valid);   // first start >= row end
    if (hi < lo) hi = lo;
    lo = min(lo, c.n_docs);
    hi = min(hi, c.n_docs);
    int64_t inner = c.nz_rank[hi] - c.nz_rank[lo];
    segs = 1 + (int32_t)inner + (valid < c.PL ? 1 : 0);
    aux = c.nz_rank[lo];
  } else {
    const int64_t n_nz = c.nz_rank[c.n_docs];
    const int64_t k0 = r * c.mb;
    if (k0 >= n_nz) {
      valid = 0;
      segs = 0;
      aux = 0;
    } else {
      const int64_t k1 = min(k0 + c.mb, n_nz);
      const int64_t start = c.trunc_scan[c.slot_doc[k0]];
      const int64_t end = k1 < n_nz ? c.trunc_scan[c.slot_doc[k1]] : c.trunc_scan[c.n_docs];
      valid = (int32_t)(end - start);
      segs = (int32_t)(k1 - k0) + (valid < c.PL ? 1 : 0);
      aux = start;
    }
  }
  c.row_valid[r] = valid;
  if (c.valid_out) c.valid_out[r] = valid;
  c.row_aux[r] = aux;
  c.row_cnt[r] = segs;
}

// One block: exclusive scan of per-row segment counts into row_seg_ptr, the
// final boundary, and the statistics header.
__global__ void __launch_bounds__(kThreads) k_row_scan(int32_t* row_seg_ptr, int64_t n_rows, int32_t PL,
                                                        int32_t* cu, int64_t cap, int32_t* stats,
                                                        const int64_t* nz_rank, int64_t n_docs, int mode,
                                                        int32_t mb) {
  __shared__ Pair lds[kThreads / 64];
  Pair carry = {0, 0};
  for (int64_t c = 0; c < n_rows; c += kThreads) {
    int64_t i = c + threadIdx.x;
    Pair v = {i < n_rows ? row_seg_ptr[i] : 0, 0};
    Pair tot;
    Pair ex = block_exclusive_scan(v, &tot, lds);
    if (i < n_rows) row_seg_ptr[i] = (int32_t)(carry.a + ex.a);
    carry = carry + tot;
  }
  if (threadIdx.x == 0) {
    const int32_t n_seg = (int32_t)carry.a;
    row_seg_ptr[n_rows] = n_seg;
    int64_t filled = mode == 0 ? n_rows : (nz_rank[n_docs] + mb - 1) / mb;
    stats[0] = n_seg;
    stats[1] = 0;
    stats[2] = (int32_t)filled;
    // stats[3] flags offsets that broke the stated precondition (the segment
    // count overran the capacity); nothing is then written past it.
    stats[3] = (n_seg < 0 || n_seg > cap) ? 1 : 0;
    if (n_seg >= 0 && n_seg <= cap) cu[n_seg] = (int32_t)(filled * PL);
  }
}

struct EmitCtx {
  int mode;
  const int32_t* tokens;
  const int64_t* off;
  int64_t n_docs, n_tokens, n_rows;
  int32_t mb, seq_len, PL;
  const int64_t *nz_rank, *trunc_scan, *slot_doc, *row_aux;
  const int32_t* row_valid;
  int32_t *ids, *labels, *indexes;
};

constexpr int kEmitRun = 4;  // consecutive output positions per thread

// Every output position: token id, label and position inside its segment.
__global__ void __launch_bounds__(kThreads) k_emit(EmitCtx c) {
  const int64_t total = c.n_rows * (int64_t)c.PL;
  const int64_t g0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kEmitRun;
  if (g0 >= total) return;
  const int64_t n_nz = c.nz_rank[c.n_docs];
  int64_t d = -1;  // carry-over: document holding the current stream position
  int64_t k = -1;  // truncate: slot (non-empty document rank) of the current position
  for (int u = 0; u < kEmitRun; ++u) {
    const int64_t g = g0 + u;
    if (g >= total) break;
    const int64_t r = g / c.PL;
    const int32_t p = (int32_t)(g - r * c.PL);
    const int32_t valid = c.row_valid[r];
    int32_t id = 0, lab = -100, idx;
    if (p >= valid) {
      // padding tail (or an unfilled row): one segment from `valid`
      idx = p - valid;
    } else if (c.mode == 0) {
      const int64_t P = g;  // stream position of this output slot
      if (d < 0) d = min(max(upper_bound(c.off, c.n_docs + 1, P) - 1, (int64_t)0), c.n_docs - 1);
      while (d + 1 < c.n_docs && clamp_off(c.off, d + 1, c.n_tokens) <= P) ++d;
      const int64_t ds = clamp_off(c.off, d, c.n_tokens);
      const int64_t de = clamp_off(c.off, d + 1, c.n_tokens);
      id = c.tokens[P];
      lab = (P + 1 < de) ? c.tokens[P + 1] : -100;
      idx = (int32_t)(P - max(ds, r * (int64_t)c.PL));
    } else {
      const int64_t k0 = r * c.mb;
      const int64_t k1 = min(k0 + c.mb, n_nz);
      const int64_t base = c.row_aux[r];
      if (k < k0 || k >= k1) {
        // last slot whose start (inside the row) is <= p
        int64_t lo = k0, hi = k1;
        while (hi - lo > 1) {
          int64_t mid = (lo + hi) >> 1;
          if (c.trunc_scan[c.slot_doc[mid]] - base <= p) lo = mid; else hi = mid;
        }
        k = lo;
      }
      while (k + 1 < k1 && c.trunc_scan[c.slot_doc[k + 1]] - base <= p) ++k;
      const int64_t dd = c.slot_doc[k];
      const int64_t local = p - (c.trunc_scan[dd] - base);
      const int64_t ds = clamp_off(c.off, dd, c.n_tokens);
      const int64_t de = clamp_off(c.off, dd + 1, c.n_tokens);
      const int64_t tlen = min(de - ds, (int64_t)c.seq_len);
      if (local >= 0 && local < tlen) {
        id = c.tokens[ds + local];
        lab = (local + 1 < tlen) ? c.tokens[ds + local + 1] : -100;
      }
      idx = (int32_t)local;
    }
    c.ids[g] = id;
    c.labels[g] = lab;
    c.indexes[g] = idx;
  }
}

struct BoundCtx {
  int mode;
  const int64_t* off;
  int64_t n_docs, n_tokens, n_rows, cap;
  int32_t mb, PL;
  const int64_t *nz_rank, *trunc_scan, *row_aux;
  const int32_t *row_valid, *row_seg_ptr;
  int32_t* cu;
};

// Threads [0, n_rows) write row starts and padding starts; threads
// [n_rows, n_rows + n_docs) write the document starts inside rows.
__global__ void __launch_bounds__(kThreads) k_bounds(BoundCtx c) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t < c.n_rows) {
    const int64_t r = t;
    const int32_t a = c.row_seg_ptr[r], b = c.row_seg_ptr[r + 1];
    if (b > a && a >= 0 && b <= c.cap) {  // filled row
      c.cu[a] = (int32_t)(r * c.PL);
      const int32_t valid = c.row_valid[r];
      if (valid < c.PL) c.cu[b - 1] = (int32_t)(r * c.PL + valid);
    }
    return;
  }
  const int64_t d = t - c.n_rows;
  if (d >= c.n_docs) return;
  const int64_t s = clamp_off(c.off, d, c.n_tokens);
  const int64_t e = clamp_off(c.off, d + 1, c.n_tokens);
  if (e <= s) return;  // empty document: no boundary
  if (c.mode == 0) {
    const int64_t r = s / c.PL;
    if (s == r * c.PL) return;  // starts a row: written by the row thread
    if (r >= c.n_rows) return;
    const int64_t slot = c.row_seg_ptr[r] + 1 + (c.nz_rank[d] - c.row_aux[r]);
    if (slot > 0 && slot < c.cap) c.cu[slot] = (int32_t)s;
  } else {
    const int64_t kk = c.nz_rank[d];
    const int64_t r = kk / c.mb;
    const int64_t j = kk - r * c.mb;
    if (j == 0 || r >= c.n_rows) return;
    const int64_t slot = c.row_seg_ptr[r] + j;
    if (slot > 0 && slot < c.cap) c.cu[slot] = (int32_t)(r * c.PL + (c.trunc_scan[d] - c.row_aux[r]));
  }
}

__global__ void __launch_bounds__(kThreads) k_max_seqlen(const int32_t* cu, int64_t cap, int32_t* stats) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int32_t n_seg = stats[0];
  int32_t v = (i < cap && i < n_seg) ? cu[i + 1] - cu[i] : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  __shared__ int32_t w[kThreads / 64];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t m = w[0];
    for (int j = 1; j < kThreads / 64; ++j) m = max(m, w[j]);
    if (m > 0) atomicMax(&stats[1], m);
  }
}

inline unsigned grid_for(int64_t n, int64_t per_block) {
  return (unsigned)((n + per_block - 1) / per_block);
}

}  // namespace

size_t pack_workspace_bytes(int64_t n_docs, int64_t n_rows) {
  const int64_t n_blocks = (n_docs + 1 + kScanTile - 1) / kScanTile;
  size_t b = 0;
  b += align_up(sizeof(int64_t) * (n_docs + 1), 256) * 2;
  b += align_up(sizeof(int64_t) * (n_docs + 1), 256);
  b += align_up(sizeof(int64_t) * 2 * n_blocks, 256);
  b += align_up(sizeof(int64_t) * (n_rows + 1), 256);
  b += align_up(sizeof(int32_t) * (n_rows + 1), 256);
  return b;
}

PackWorkspace pack_carve(void* ws, int64_t n_docs, int64_t n_rows) {
  PackWorkspace w;
  char* p = static_cast<char*>(ws);
  w.n_blocks = (n_docs + 1 + kScanTile - 1) / kScanTile;
  w.nz_rank = reinterpret_cast<int64_t*>(p); p += align_up(sizeof(int64_t) * (n_docs + 1), 256);
  w.trunc_scan = reinterpret_cast<int64_t*>(p); p += align_up(sizeof(int64_t) * (n_docs + 1), 256);
  w.slot_doc = reinterpret_cast<int64_t*>(p); p += align_up(sizeof(int64_t) * (n_docs + 1), 256);
  w.partials = reinterpret_cast<int64_t*>(p); p += align_up(sizeof(int64_t) * 2 * w.n_blocks, 256);
  w.row_aux = reinterpret_cast<int64_t*>(p); p += align_up(sizeof(int64_t) * (n_rows + 1), 256);
  w.row_valid = reinterpret_cast<int32_t*>(p);
  return w;
}

hipError_t launch_pack(const PackArgs& a, hipStream_t stream) {
  ScopedKernelTimer timed(kTimePack, stream);
  PackWorkspace w = pack_carve(a.workspace, a.n_docs, a.n_rows);
  const unsigned nb = (unsigned)w.n_blocks;
  k_scan_partial<<<nb, kThreads, 0, stream>>>(a.doc_offsets, a.n_docs, a.n_tokens, a.seq_len, w.partials);
  k_scan_top<<<1, kThreads, 0, stream>>>(w.partials, w.n_blocks);
  k_scan_final<<<nb, kThreads, 0, stream>>>(a.doc_offsets, a.n_docs, a.n_tokens, a.seq_len, w.partials,
                                            w.nz_rank, w.trunc_scan, w.slot_doc);
  if (a.n_rows > 0) {
    RowCtx rc{a.mode, a.doc_offsets, a.n_docs, a.n_tokens, a.n_rows, a.micro_bsz, a.seq_len,
              a.packed_length, w.nz_rank, w.trunc_scan, w.slot_doc, w.row_aux, w.row_valid,
              a.row_seg_ptr, a.row_valid_len};
    k_row_count<<<grid_for(a.n_rows, kThreads), kThreads, 0, stream>>>(rc);
  }
  k_row_scan<<<1, kThreads, 0, stream>>>(a.row_seg_ptr, a.n_rows, a.packed_length, a.cu_seqlens,
                                         a.max_segments, a.stats, w.nz_rank, a.n_docs, a.mode, a.micro_bsz);
  if (a.n_rows > 0) {
    EmitCtx ec{a.mode, a.tokens, a.doc_offsets, a.n_docs, a.n_tokens, a.n_rows, a.micro_bsz, a.seq_len,
               a.packed_length, w.nz_rank, w.trunc_scan, w.slot_doc, w.row_aux, w.row_valid,
               a.input_ids, a.labels, a.indexes};
    const int64_t total = a.n_rows * (int64_t)a.packed_length;
    k_emit<<<grid_for(total, (int64_t)kThreads * kEmitRun), kThreads, 0, stream>>>(ec);
    BoundCtx bc{a.mode, a.doc_offsets, a.n_docs, a.n_tokens, a.n_rows, a.max_segments, a.micro_bsz,
                a.packed_length,
                w.nz_rank, w.trunc_scan, w.row_aux, w.row_valid, a.row_seg_ptr, a.cu_seqlens};
    k_bounds<<<grid_for(a.n_rows + a.n_docs, kThreads), kThreads, 0, stream>>>(bc);
    k_max_seqlen<<<grid_for(a.max_segments, kThreads), kThreads, 0, stream>>>(a.cu_seqlens, a.max_segments,
                                                                               a.stats);
  }
  return hipGetLastError();
}

}  // namespace psc
