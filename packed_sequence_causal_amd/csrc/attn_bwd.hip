// Document-causal attention backward, bf16 operands / fp32 accumulate, gfx950.
//
// Gradients of sum(dO * O) for O = softmax(scale * Q K^T restricted to each
// document's causal triangle) V, with P recomputed from the forward's lse:
//   D_i   = <dO_i, O_i>                      (in k_bwd_dq, stored negated with
//                                              -lse_i / scale for k_bwd_dkdv,
//                                              which runs after it: the two
//                                              start the dP and S accumulators)
//   P     = exp(scale * q_i.k_j - lse_i)      (recomputed, exp2 domain)
//   dP    = dO V^T,   dS = P * (dP - D)
//   dV    = P^T dO,   dK = scale dS^T Q       (k_bwd_dkdv, D = 64, and
//                                              k_bwd_dkdv8, D = 128: one
//                                              workgroup per 128-key tile and
//                                              key/value head; loops over the
//                                              head group's query heads and the
//                                              query blocks from the tile to
//                                              the document end)
//   dQ    = scale dS K                        (k_bwd_dq: one workgroup per
//                                              query tile and group of HP query
//                                              heads sharing a key/value head,
//                                              128 / HP rows; loops over key
//                                              blocks up to the diagonal)
// Splitting dQ from dK/dV recomputes S and dP once more but needs no atomics:
// every output element is written once, and results are deterministic.
// Both loops visit only tiles inside a document's causal triangle ("Sample
// Packing：长序列 LLM 训练的 Attention 问题及优化", section 5.1).
//
// The streamed operand of each kernel (K/V blocks for dQ, Q/dO blocks plus
// their lse and D for dK/dV) is double-buffered in LDS and filled with
// asynchronous direct-to-LDS loads, as in the forward (attn_common.h).
#include <type_traits>

#include "attn_common.h"
#include "psc_internal.h"
#include "rope_common.h"

namespace psc {
namespace {

constexpr int kThreads = 256;
constexpr int kBQ = 128;   // dQ kernel: query rows x heads per workgroup (4 waves x 32 rows)
constexpr int kBNq = 64;   // dQ kernel: keys per block
constexpr int kBKV = 128;  // dK/dV kernel: keys per workgroup (4 waves x 32)
constexpr int kBMk = 64;   // dK/dV kernel: queries per block
constexpr int kDkdvValuPerMfma = 4;  // VALU instructions placed after each MFMA of the softmax regions
constexpr int kDqValuPerMfma = 3;    // dQ kernel: VALU instructions after each MFMA of its mixed region

struct BwdParams {
  const bf16 *q, *k, *v, *o, *dout;
  const float* lse;
  float* Dbuf;   // [hq][T]  -D_i
  float* NLbuf;  // [hq][T]  -lse_i / scale
  void *dq, *dk, *dv;  // float32, or bf16 when grad_bf16
  int64_t sq, sk, sv, so, sdo, T;
  const int32_t* cu;
  const int32_t* items;
  const int32_t* n_items;
  int32_t hq, hkv, group;
  float scale, scale_log2;
  int32_t grad_bf16;  // launch selection only: the kernels take it as a template parameter
  // rotary embedding (the ROPE instantiations only): q and k arrive turned,
  // and dq, dk are turned back by -theta before they are stored
  const int32_t* pos;     // [T] position of each token
  const float2* rope_cs;  // [rope_n_pos][D/2] (cos, sin)
  int32_t rope_n_pos;
};

// (cos, sin) of the turn at token t (position clamped to the table).
__device__ __forceinline__ const float2* rope_row(const BwdParams& p, int64_t t, int half) {
  return p.rope_cs + (int64_t)min(max(p.pos[t], 0), p.rope_n_pos - 1) * half;
}

// ---------------------------------------------------------------------- dQ

template <int D>
struct DqState {
  bf16x8 qf[D / 16], df[D / 16];
  f32x16 acc[D / 32];
  float lse2, Drow;
};

// Keeps the computation of x before this point (IR passes otherwise sink
// arithmetic past a scheduling barrier, next to its first use).
__device__ __forceinline__ void pin(bf16x8& x) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  i32x4 t = __builtin_bit_cast(i32x4, x);
  asm volatile("" : "+v"(t));
  x = __builtin_bit_cast(bf16x8, t);
}

// One 64-key block of the dQ loop for one wave, in two 32-key halves so that
// the VALU work of one half sits in the same basic block as MFMAs of the
// other (a diagonal block's mask is a uniform branch, which ends a block):
//   S, dP of half 0 | [mask 0] | S, dP of half 1 + dS of half 0 (scheduled
//   together) | [mask 1] |
//   dS of half 1 + dQ products
template <int D>
__device__ __forceinline__ void dq_block(DqState<D>& st, const char* Ks, const char* Vs, int32_t kb, int32_t L,
                                         int32_t qrow, int32_t wq_lo, float c2, int h, int lq, int l) {
  const char* Kb = reinterpret_cast<const char*>(Ks);
  const char* Vb = reinterpret_cast<const char*>(Vs);
  const bool diag = (kb + kBNq - 1 > wq_lo) || (kb + kBNq > L);
  // key kb + 32 n2 + 8 (i / 4) + 4 h + i % 4 is masked when it is after the
  // row or at/after the document end: one compare with a constant per score
  const int32_t lim = min(qrow + 1, L) - kb - 4 * h;
  const float neg_l = -st.lse2;
  auto sdp = [&](int n2, f32x16& sa, f32x16& da) {
    sa = f32x16{};
    da = f32x16{};
    const int r = 32 * n2 + lq;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8 ak = *reinterpret_cast<const bf16x8*>(Kb + lds_byte(r, 16 * kk + 8 * h));
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(Vb + lds_byte(r, 16 * kk + 8 * h));
      sa = mfma32(ak, st.qf[kk], sa);
      da = mfma32(av, st.df[kk], da);
    }
  };
  auto mask = [&](int n2, f32x16& sa) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (32 * n2 + 8 * (i >> 2) + (i & 3) >= lim) sa[i] = -INFINITY;
    }
  };
  auto ds = [&](const f32x16& sa, const f32x16& da, bf16x8* out) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pr = fast_exp2(__builtin_fmaf(sa[i], c2, neg_l));
      out[i >> 3][i & 7] = (bf16)(pr * (da[i] - st.Drow));
    }
  };
  f32x16 s0, dp0, s1, dp1;
  bf16x8 dsb[4];
  sdp(0, s0, dp0);
  if (diag) mask(0, s0);
  // region: S, dP of half 1 (16 MFMAs, 16 row reads) + dS of half 0 (VALU)
  sdp(1, s1, dp1);
  ds(s0, dp0, dsb);
  PSC_SCHED_DS_READ(2);
#pragma unroll
  for (int i = 0; i < 2 * (D / 16); ++i) {
    PSC_SCHED_MFMA(1);
    if (i < 2 * (D / 16) - 2) PSC_SCHED_DS_READ(1);
    PSC_SCHED_VALU(kDqValuPerMfma);
  }
  pin(dsb[0]);
  pin(dsb[1]);
  __builtin_amdgcn_sched_barrier(0);
  if (diag) mask(1, s1);
  // region: dS of half 1 + dQ products (those of half 0 first)
  ds(s1, dp1, dsb + 2);
  // (addresses from lds_byte here: the shared TileReadOffsets bases made this
  // kernel's schedule slower)
  const int gi = l & 15;
  const int dsub = 16 * ((l >> 4) & 1);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int col = 32 * dt + dsub + 4 * (gi & 3);
      const int r0 = 16 * ks + 4 * h + (gi >> 2);
      const bf16* p0 = reinterpret_cast<const bf16*>(Kb + lds_byte(r0, col));
      const bf16* p1 = reinterpret_cast<const bf16*>(Kb + lds_byte(r0 + 8, col));
      st.acc[dt] = mfma32(tr_read8(p0, p1), dsb[ks], st.acc[dt]);
    }
  }
}

// HP query heads of one key/value group per workgroup (1, 2 or 4), each on
// 128 / HP rows: wave w takes head w % HP and rows 32 (w / HP) .. +31 of the
// tile, so with HP = 4 all four waves cover the same rows (equal work) and
// share every key/value block.
// DR = D / 2 runs heads of DR columns in the D-column kernel (as in the
// forward): Q and dO are zero past DR in registers, so S, dP and D_i are those
// of the head's columns, and only dQ's first DR columns are stored.
// GB: dQ stored in bf16 (else fp32); a template parameter so the fp32
// kernel's code and registers are those of a kernel with no bf16 path.
template <int D, int HP, int DR = D, bool GB = false, bool ROPE = false>
__global__ void __launch_bounds__(kThreads, 2) k_bwd_dq(BwdParams p) {
  static_assert(DR == D || 2 * DR == D, "a head fills the tile or half of it");
  constexpr int RW = kBQ / HP;  // query rows per workgroup
  __shared__ __attribute__((aligned(16))) char Ks0[tile_bytes<D>()];
  __shared__ __attribute__((aligned(16))) char Vs0[tile_bytes<D>()];
  __shared__ __attribute__((aligned(16))) char Ks1[tile_bytes<D>()];
  __shared__ __attribute__((aligned(16))) char Vs1[tile_bytes<D>()];

  const int tid = threadIdx.x, l = tid & 63, h = l >> 5, lq = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t ngrp = (uint32_t)(p.hq / HP);  // workgroups per tile
  const uint32_t b = xcd_group_remap(blockIdx.x, gridDim.x, (uint32_t)(p.group / HP));
  const uint32_t item = b / ngrp, hg = b % ngrp;
  const int hw = w % HP, rs = w / HP;
  const int32_t head = (int32_t)hg * HP + hw;
  // item < cap (the grid is cap work-groups per head group), so the entry is read
  // together with the count and used only once the count admits it.  The
  // schedule writes every entry below the count, with segment bounds clamped
  // to [0, T]: a malformed cu_seqlens cannot send any access outside the
  // tensors.
  const int4 it = *reinterpret_cast<const int4*>(p.items + 4 * item);
  if ((int32_t)item >= *p.n_items) return;
  const int32_t s0 = it.x, L = it.y, tile = it.z;
  const int32_t q0 = tile * RW;
  if (q0 >= L) return;
  const int32_t kvh = (int32_t)hg * HP / p.group;

  const bf16* Kp = p.k + (int64_t)s0 * p.sk + (int64_t)kvh * DR;
  const bf16* Vp = p.v + (int64_t)s0 * p.sv + (int64_t)kvh * DR;
  const int32_t kv_end = min(q0 + RW, L);
  const int32_t nkv = (kv_end + kBNq - 1) / kBNq;
  uint32_t koff[D / 8 / (kThreads / 64)], voff[D / 8 / (kThreads / 64)];
  tile_offsets<D, kThreads / 64, DR>(p.sk, w, l, koff);
  tile_offsets<D, kThreads / 64, DR>(p.sv, w, l, voff);
  load_tile<D, kThreads / 64, DR>(Kp, p.sk, 0, L, koff, Ks0, w, l);
  load_tile<D, kThreads / 64, DR>(Vp, p.sv, 0, L, voff, Vs0, w, l);

  const int32_t qrow = q0 + 32 * rs + lq;
  const bool qvalid = qrow < L;
  DqState<D> st;
  // the row's rotary position, fetched before the key loop so the epilogue
  // waits on one load (the table row), not on two in a chain
  int32_t rope_pos = 0;
  if constexpr (ROPE) rope_pos = qvalid ? min(max(p.pos[s0 + qrow], 0), p.rope_n_pos - 1) : 0;
  {
    const bf16* Qr = p.q + (int64_t)(s0 + qrow) * p.sq + (int64_t)head * DR;
    const bf16* Dr = p.dout + (int64_t)(s0 + qrow) * p.sdo + (int64_t)head * DR;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bool in = qvalid && 16 * kk + 8 * h < DR;
      st.qf[kk] = in ? *reinterpret_cast<const bf16x8*>(Qr + 16 * kk + 8 * h) : bf16x8{};
      st.df[kk] = in ? *reinterpret_cast<const bf16x8*>(Dr + 16 * kk + 8 * h) : bf16x8{};
    }
  }
  // D_i = <dO_i, O_i> from the dO fragments already held (lanes l and l ^ 32
  // hold the two halves of row lq) and the same fragments of O; -D and
  // -lse / scale are also stored for the dK/dV kernel, which runs next.  The
  // tiles partition every document, so each (row, head) is written once.
  {
    float dacc = 0.f;
    if (qvalid) {
      const bf16* Or = p.o + (int64_t)(s0 + qrow) * p.so + (int64_t)head * DR;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        if (16 * kk + 8 * h >= DR) continue;
        const bf16x8 of = *reinterpret_cast<const bf16x8*>(Or + 16 * kk + 8 * h);
#pragma unroll
        for (int e = 0; e < 8; ++e) dacc = __builtin_fmaf((float)of[e], (float)st.df[kk][e], dacc);
      }
    }
    st.Drow = sum_halves(dacc);
    st.lse2 = qvalid ? p.lse[(int64_t)head * p.T + s0 + qrow] * kLog2e : 0.f;
    if (qvalid && h == 0) {
      p.Dbuf[(int64_t)head * p.T + s0 + qrow] = -st.Drow;
      p.NLbuf[(int64_t)head * p.T + s0 + qrow] = -p.lse[(int64_t)head * p.T + s0 + qrow] / p.scale;
    }
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.acc[dt] = f32x16{};

  const int32_t wq_lo = q0 + 32 * rs, wq_hi = wq_lo + 31;
  // no key blocks for a wave whose rows are all past the document end
  const int32_t wq_top = wq_lo < L ? wq_hi : -1;
  const float c2 = p.scale_log2;
  for (int32_t j = 0; j < nkv; j += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < nkv) {
      load_tile<D, kThreads / 64, DR>(Kp, p.sk, (j + 1) * kBNq, L, koff, Ks1, w, l);
      load_tile<D, kThreads / 64, DR>(Vp, p.sv, (j + 1) * kBNq, L, voff, Vs1, w, l);
    }
    if (j * kBNq <= wq_top) dq_block<D>(st, Ks0, Vs0, j * kBNq, L, qrow, wq_lo, c2, h, lq, l);
    if (j + 1 >= nkv) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 2 < nkv) {
      load_tile<D, kThreads / 64, DR>(Kp, p.sk, (j + 2) * kBNq, L, koff, Ks0, w, l);
      load_tile<D, kThreads / 64, DR>(Vp, p.sv, (j + 2) * kBNq, L, voff, Vs0, w, l);
    }
    if ((j + 1) * kBNq <= wq_top) dq_block<D>(st, Ks1, Vs1, (j + 1) * kBNq, L, qrow, wq_lo, c2, h, lq, l);
  }

  // Epilogue: dQ goes out through LDS so that each store instruction writes
  // whole runs of 64 lanes x 16 bytes (4 rows) instead of 32-byte pieces of
  // 32 rows.  The stage the last block did not use is free (its block was
  // consumed before the last barrier, and no load targets it); each wave
  // stages its 32 rows in its own half of one of its tiles, kPW columns at a
  // time.  Inside a staged row, 16-byte chunk c sits at slot c ^ (row % kPC).
  char* const stage = (nkv & 1) ? (w < 2 ? Ks1 : Vs1) : (w < 2 ? Ks0 : Vs0);
  char* const ob = stage + (w & 1) * (tile_bytes<D>() / 2);
  float omul = p.scale;
  if constexpr (ROPE) {
    // dQ of the turned q, scaled, turned back by -theta: register i of acc[dt]
    // is dim 32 dt + 8 (i / 4) + 4 h + i % 4 of the lane's row, so dims d and
    // d + D/2 are acc[dt] and acc[dt + D/64] of the same lane and register
    static_assert(DR == D, "the turn pairs registers of one lane");
    constexpr int HD = D / 64;
    if (qvalid) {
      const float2* cs = p.rope_cs + (int64_t)rope_pos * (D / 2);
#pragma unroll
      for (int dt = 0; dt < HD; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4* c4 = reinterpret_cast<const float4*>(cs + 32 * dt + 8 * g + 4 * h);
          const float4 t0 = c4[0], t1 = c4[1];
          const float cc[4] = {t0.x, t0.z, t1.x, t1.z}, ss[4] = {t0.y, t0.w, t1.y, t1.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float y1, y2;
            rope_turn(st.acc[dt][4 * g + e] * p.scale, st.acc[dt + HD][4 * g + e] * p.scale, cc[e], -ss[e], y1, y2);
            st.acc[dt][4 * g + e] = y1;
            st.acc[dt + HD][4 * g + e] = y2;
          }
        }
      }
    }
    omul = 1.f;
  }
  if constexpr (GB) {
    // bf16 dQ: whole 2*D-byte rows fit half a tile at once (as the forward's O)
    constexpr int kChunks = D / 8;
    bf16* const dq = static_cast<bf16*>(p.dq);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (bf16)(st.acc[dt][4 * g4 + e] * omul);
        const int c = 4 * dt + g4;
        *reinterpret_cast<bf16x4*>(ob + lq * (2 * D) + ((c ^ (lq & (kChunks - 1))) << 4) + 8 * h) = o4;
      }
    }
    constexpr int kRowsPerStore = 64 / kChunks;
    const int c = l % kChunks;
#pragma unroll
    for (int k = 0; k < 32 / kRowsPerStore; ++k) {
      const int r = k * kRowsPerStore + l / kChunks;
      const bf16x8 v8 = *reinterpret_cast<const bf16x8*>(ob + r * (2 * D) + ((c ^ (r & (kChunks - 1))) << 4));
      const int32_t row = wq_lo + r;
      if (row < L && 8 * c < DR) *reinterpret_cast<bf16x8*>(dq + ((int64_t)(s0 + row) * p.hq + head) * DR + 8 * c) = v8;
    }
  } else {
    constexpr int kPW = tile_bytes<D>() / 256;  // fp32 columns per pass: 32 rows x kPW x 4 B = half a tile
    constexpr int kPC = kPW / 4;                 // 16-byte chunks per staged row
    static_assert(DR % kPW == 0, "passes cover whole heads");
    float* const dq = static_cast<float*>(p.dq);
#pragma unroll
    for (int pass = 0; pass < DR / kPW; ++pass) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        if ((32 * dt) / kPW != pass) continue;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = st.acc[dt][4 * g4 + e] * omul;
          const int c = (32 * dt - kPW * pass) / 4 + 2 * g4 + h;
          *reinterpret_cast<f32x4*>(ob + lq * (4 * kPW) + ((c ^ (lq & (kPC - 1))) << 4)) = v4;
        }
      }
      constexpr int kRowsPerStore = 64 / kPC;
      const int c = l % kPC;
#pragma unroll
      for (int k = 0; k < 32 / kRowsPerStore; ++k) {
        const int r = k * kRowsPerStore + l / kPC;
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(ob + r * (4 * kPW) + ((c ^ (r & (kPC - 1))) << 4));
        const int32_t row = wq_lo + r;
        if (row < L) *reinterpret_cast<f32x4*>(dq + ((int64_t)(s0 + row) * p.hq + head) * DR + kPW * pass + 4 * c) = v4;
      }
    }
  }
}

// ------------------------------------------------------------------ dK, dV

template <int D>
struct DkvState {
  bf16x8 kf[D / 16], vf[D / 16];
  f32x16 dka[D / 32], dva[D / 32];
};

// One 64-query block of the four-wave dK/dV loop for one wave (keys wk_lo ..
// +31, this lane's key `key`), software-pipelined inside the wave (a wave's own
// instruction stream has to hide most of its latencies).  Blocks on the
// diagonal or at the document end (MASK) take the same schedule with the
// mask applied to S just before B; a half whose queries all precede the
// wave's keys is computed and then fully masked (cheaper than a separate,
// unscheduled path).  Per 32-query half mq the work is
//   A(mq): S and dP (16 MFMAs, operand rows read from LDS)
//   B(mq): P and dS in bf16, laid out as the A operand of the next products
//   C(mq): dV += P^T dO and dK += dS^T Q (16 MFMAs, column reads from LDS)
// issued as four regions, B split into its two 16-query slices a and b:
//   A(0) | A(1) + B(0)a | C(0) + B(0)b + B(1)a | C(1) + B(1)b
// so that the VALU work of one half runs between the MFMAs of the other (the
// C MFMAs of slice a go first, those of slice b after its B part).  Each
// region ends by reading the first operands of the next one.
#define PSC_SCHED_BARRIER() __builtin_amdgcn_sched_barrier(0)

__device__ __forceinline__ bf16x8 ld8(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }


// Scores of query half qm (queries qm + 8 (i / 4) + 4 h + i % 4 of register
// i) before this lane's key or at/after the document end get -inf.
__device__ __forceinline__ void mask_half(f32x16& s, int32_t qm, int32_t key, int32_t L, int h) {
  const int32_t lo = key - qm - 4 * h, hi = L - qm - 4 * h;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = 8 * (i >> 2) + (i & 3);
    if (c < lo || c >= hi) s[i] = -INFINITY;
  }
}

template <int D, bool MASK>
__device__ __forceinline__ void dkdv_block_full(DkvState<D>& st, const char* Qs, const char* dOs, const float* NLs,
                                                const float* Ds, float c2, int h, const TileReadOffsets& o,
                                                int32_t qs, int32_t key, int32_t L) {
  constexpr int KS = D / 16;
  constexpr int NC = D / 16;
  constexpr int PF = 3;  // operands of the next region read ahead
  // A operand of S/dP: row 32*mq + lq, k-step kk
  auto offA = [&](int mq, int kk) { return row_off(o, kk) + mq * 32 * 128; };
  // B operand of dV/dK, pair c = ks * (D/32) + dt: column read of rows 32*mq + 16*ks ..
  auto trC = [&](const char* M, int mq, int c) { return col_operand(M + mq * 32 * 128, o, c / (D / 32), c % (D / 32)); };
  // s already holds S - lse / scale and dp holds dP - D: their accumulators
  // start from -lse / scale and -D (see below)
  auto pds = [&](const f32x16& s, const f32x16& dp, bf16x8* pa, bf16x8* da, int i0 = 0, int i1 = 16) {
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const float pr = fast_exp2(s[i] * c2);
      pa[i >> 3][i & 7] = (bf16)pr;
      da[i >> 3][i & 7] = (bf16)(pr * dp[i]);
    }
  };
  // values of this lane's 16 query rows of half mq (register i <-> query
  // 8 (i / 4) + 4 h + i % 4): -D and -lse / scale, the starting values of
  // the dP and S accumulators
  auto rows16 = [&](const float* vec, int mq) {
    f32x16 r;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(vec + 32 * mq + 8 * g + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) r[4 * g + e] = v[e];
    }
    return r;
  };

  // ---------------- region 1: A(0)
  f32x16 s0 = rows16(NLs, 0), s1;
  f32x16 dp0 = rows16(Ds, 0);
  f32x16 dp1;
  bf16x8 nq[KS], nd[KS];        // A(1) operands
  {
    bf16x8 aq[KS], ad[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      aq[kk] = ld8(Qs + offA(0, kk));
      ad[kk] = ld8(dOs + offA(0, kk));
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      s0 = mfma32(aq[kk], st.kf[kk], s0);
      dp0 = mfma32(ad[kk], st.vf[kk], dp0);
    }
    s1 = rows16(NLs, 1);
    dp1 = rows16(Ds, 1);
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) {
      nq[kk] = ld8(Qs + offA(1, kk));
      nd[kk] = ld8(dOs + offA(1, kk));
    }
    // -D and eight operand reads ahead of the first MFMA, then one per MFMA
    PSC_SCHED_DS_READ(12);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      PSC_SCHED_MFMA(1);
      if (i < 2 * KS - 4) PSC_SCHED_DS_READ(1);
    }
    PSC_SCHED_DS_READ(8 + 4 + 2 * PF);
  }
  PSC_SCHED_BARRIER();
  // ---------------- region 2: A(1) + B(0)a
  bf16x8 pa0[2], da0[2];
  bf16x8 cb[PF], cq[PF];        // C(0) operands
  {
#pragma unroll
    for (int kk = PF; kk < KS; ++kk) {
      nq[kk] = ld8(Qs + offA(1, kk));
      nd[kk] = ld8(dOs + offA(1, kk));
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      s1 = mfma32(nq[kk], st.kf[kk], s1);
      dp1 = mfma32(nd[kk], st.vf[kk], dp1);
    }
    if (MASK) mask_half(s0, qs, key, L, h);
    pds(s0, dp0, pa0, da0, 0, 8);
#pragma unroll
    for (int c = 0; c < PF; ++c) {
      cb[c] = trC(dOs, 0, c);
      cq[c] = trC(Qs, 0, c);
    }
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      PSC_SCHED_MFMA(1);
      PSC_SCHED_DS_READ(1);
      PSC_SCHED_VALU(kDkdvValuPerMfma);
    }
    PSC_SCHED_DS_READ(8 + 4 * PF);
  }
  pin(pa0[0]); pin(da0[0]);
  PSC_SCHED_BARRIER();
  // ---------------- region 3: C(0) + B(0)b + B(1)a
  bf16x8 pa1[2], da1[2];
  bf16x8 eb[PF], eq[PF];        // C(1) operands
  {
    bf16x8 bo[NC], bq[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bo[c] = c < PF ? cb[c] : trC(dOs, 0, c);
      bq[c] = c < PF ? cq[c] : trC(Qs, 0, c);
    }
#pragma unroll
    for (int c = 0; c < NC / 2; ++c) {
      const int dt = c % (D / 32);
      st.dva[dt] = mfma32(pa0[0], bo[c], st.dva[dt]);
      st.dka[dt] = mfma32(da0[0], bq[c], st.dka[dt]);
    }
    pds(s0, dp0, pa0, da0, 8, 16);
#pragma unroll
    for (int c = NC / 2; c < NC; ++c) {
      const int dt = c % (D / 32);
      st.dva[dt] = mfma32(pa0[1], bo[c], st.dva[dt]);
      st.dka[dt] = mfma32(da0[1], bq[c], st.dka[dt]);
    }
    if (MASK) mask_half(s1, qs + 32, key, L, h);
    pds(s1, dp1, pa1, da1, 0, 8);
#pragma unroll
    for (int c = 0; c < PF; ++c) {
      eb[c] = trC(dOs, 1, c);
      eq[c] = trC(Qs, 1, c);
    }
#pragma unroll
    for (int i = 0; i < 2 * NC; ++i) {
      PSC_SCHED_MFMA(1);
      PSC_SCHED_DS_READ(2);
      PSC_SCHED_VALU(kDkdvValuPerMfma);
    }
  }
  pin(pa1[0]); pin(da1[0]);
  PSC_SCHED_BARRIER();
  // ---------------- region 4: C(1) + B(1)b
  {
    bf16x8 bo[NC], bq[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bo[c] = c < PF ? eb[c] : trC(dOs, 1, c);
      bq[c] = c < PF ? eq[c] : trC(Qs, 1, c);
    }
#pragma unroll
    for (int c = 0; c < NC / 2; ++c) {
      const int dt = c % (D / 32);
      st.dva[dt] = mfma32(pa1[0], bo[c], st.dva[dt]);
      st.dka[dt] = mfma32(da1[0], bq[c], st.dka[dt]);
    }
    pds(s1, dp1, pa1, da1, 8, 16);
#pragma unroll
    for (int c = NC / 2; c < NC; ++c) {
      const int dt = c % (D / 32);
      st.dva[dt] = mfma32(pa1[1], bo[c], st.dva[dt]);
      st.dka[dt] = mfma32(da1[1], bq[c], st.dka[dt]);
    }
    PSC_SCHED_DS_READ(4);
#pragma unroll
    for (int i = 0; i < 2 * NC; ++i) {
      PSC_SCHED_MFMA(1);
      PSC_SCHED_DS_READ(2);
      if (i < NC) PSC_SCHED_VALU(2 * kDkdvValuPerMfma);
    }
  }
  PSC_SCHED_BARRIER();
}

// D = 64 only (two waves per SIMD).  At D = 128 the K, V operands and dK, dV
// accumulators of 32 keys need ~360 registers, one wave per SIMD, and the
// eight-wave kernel below runs instead.
// DR = D / 2 runs heads of DR columns: K and V are zero past DR in registers
// (S and dP are those of the head's columns), and only the first DR columns of
// dK and dV are stored.
template <int D, int DR = D, bool GB = false, bool ROPE = false>
__global__ void __launch_bounds__(kThreads, 2) k_bwd_dkdv(BwdParams p) {
  static_assert(D == 64, "k_bwd_dkdv8 handles D = 128");
  static_assert(DR == D || 2 * DR == D, "a head fills the tile or half of it");
  __shared__ __attribute__((aligned(16))) char Qs0[tile_bytes<D>()];
  __shared__ __attribute__((aligned(16))) char dOs0[tile_bytes<D>()];
  __shared__ __attribute__((aligned(16))) char Qs1[tile_bytes<D>()];
  __shared__ __attribute__((aligned(16))) char dOs1[tile_bytes<D>()];
  __shared__ __attribute__((aligned(16))) float NLs0[kBMk];
  __shared__ __attribute__((aligned(16))) float Ds0[kBMk];
  __shared__ __attribute__((aligned(16))) float NLs1[kBMk];
  __shared__ __attribute__((aligned(16))) float Ds1[kBMk];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, lq = l & 31;
  const uint32_t item = blockIdx.x / (uint32_t)p.hkv, kvh = blockIdx.x % (uint32_t)p.hkv;
  // item < cap (the grid is cap work-groups per head), so the entry is read
  // together with the count and used only once the count admits it.  The
  // schedule writes every entry below the count, with segment bounds clamped
  // to [0, T]: a malformed cu_seqlens cannot send any access outside the
  // tensors.
  const int4 it = *reinterpret_cast<const int4*>(p.items + 4 * item);
  if ((int32_t)item >= *p.n_items) return;
  const int32_t s0 = it.x, L = it.y, tile = it.z;
  const int32_t kb = tile * kBKV;
  if (kb >= L) return;
  const int32_t key = kb + 32 * w + lq;  // this lane's key (S layout: lane <-> key)
  const bool kvalid = key < L;
  const int32_t wk_lo = kb + 32 * w;
  const int32_t nqb = (L - kb + kBMk - 1) / kBMk;
  const int32_t niter = p.group * nqb;

  uint32_t qoff[D / 8 / (kThreads / 64)], ooff[D / 8 / (kThreads / 64)];
  tile_offsets<D, kThreads / 64, DR>(p.sq, w, l, qoff);
  tile_offsets<D, kThreads / 64, DR>(p.sdo, w, l, ooff);
  // iteration t: query head kvh*G + t / nqb, query block kb + (nqb - 1 - t % nqb) * 64.
  // Blocks run from the document end back to the tile: every tile of a
  // document starts at the same rows, so tiles of one document that run at
  // the same time read the same Q/dO blocks together and L2 serves the rest.
  auto issue = [&](int32_t t, char* Qs, char* dOs, float* NLs, float* Ds) {
    const int32_t head = kvh * p.group + t / nqb;
    const int32_t qs = kb + (nqb - 1 - t % nqb) * kBMk;
    load_tile<D, kThreads / 64, DR>(p.q + (int64_t)s0 * p.sq + (int64_t)head * DR, p.sq, qs, L, qoff, Qs, w, l);
    load_tile<D, kThreads / 64, DR>(p.dout + (int64_t)s0 * p.sdo + (int64_t)head * DR, p.sdo, qs, L, ooff, dOs, w, l);
    if (w == 0) load_vec64_async(p.NLbuf + (int64_t)head * p.T + s0, qs, L, NLs, l);
    if (w == 1) load_vec64_async(p.Dbuf + (int64_t)head * p.T + s0, qs, L, Ds, l);
  };
  issue(0, Qs0, dOs0, NLs0, Ds0);

  DkvState<D> st;
  {
    const bf16* Kr = p.k + (int64_t)(s0 + key) * p.sk + (int64_t)kvh * DR;
    const bf16* Vr = p.v + (int64_t)(s0 + key) * p.sv + (int64_t)kvh * DR;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bool in = kvalid && 16 * kk + 8 * h < DR;
      st.kf[kk] = in ? *reinterpret_cast<const bf16x8*>(Kr + 16 * kk + 8 * h) : bf16x8{};
      st.vf[kk] = in ? *reinterpret_cast<const bf16x8*>(Vr + 16 * kk + 8 * h) : bf16x8{};
    }
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    st.dka[dt] = f32x16{};
    st.dva[dt] = f32x16{};
  }
  const float c2 = p.scale_log2;
  const TileReadOffsets ro = tile_read_offsets(h, lq, l);

  for (int32_t t = 0; t < niter; t += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < niter) issue(t + 1, Qs1, dOs1, NLs1, Ds1);
    {
      const int32_t qs = kb + (nqb - 1 - t % nqb) * kBMk;
      if (qs >= wk_lo + 31 && qs + kBMk <= L)
        dkdv_block_full<D, false>(st, Qs0, dOs0, NLs0, Ds0, c2, h, ro, qs, key, L);
      else if (qs + kBMk - 1 >= wk_lo && wk_lo < L)
        dkdv_block_full<D, true>(st, Qs0, dOs0, NLs0, Ds0, c2, h, ro, qs, key, L);
    }
    if (t + 1 >= niter) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 2 < niter) issue(t + 2, Qs0, dOs0, NLs0, Ds0);
    {
      const int32_t qs = kb + (nqb - 1 - (t + 1) % nqb) * kBMk;
      if (qs >= wk_lo + 31 && qs + kBMk <= L)
        dkdv_block_full<D, false>(st, Qs1, dOs1, NLs1, Ds1, c2, h, ro, qs, key, L);
      else if (qs + kBMk - 1 >= wk_lo && wk_lo < L)
        dkdv_block_full<D, true>(st, Qs1, dOs1, NLs1, Ds1, c2, h, ro, qs, key, L);
    }
  }

  // dka/dva C layout: key = wk_lo + 8*(i/4) + 4*h + i%4, d = 32*dt + lq
  float kmul = p.scale;
  if constexpr (ROPE) {
    // dK of the turned k, scaled, turned back by -theta: dims d and d + D/2 of
    // a key are dka[dt] and dka[dt + D/64] of the same lane and register
    static_assert(DR == D, "the turn pairs registers of one lane");
    constexpr int HD = D / 64;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int32_t kr = wk_lo + 8 * (i >> 2) + 4 * h + (i & 3);
      if (kr < L) {
        const float2* cs = rope_row(p, s0 + kr, D / 2);
#pragma unroll
        for (int dt = 0; dt < HD; ++dt) {
          const float2 t = cs[32 * dt + lq];
          float y1, y2;
          rope_turn(st.dka[dt][i] * p.scale, st.dka[dt + HD][i] * p.scale, t.x, -t.y, y1, y2);
          st.dka[dt][i] = y1;
          st.dka[dt + HD][i] = y2;
        }
      }
    }
    kmul = 1.f;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int32_t kr = wk_lo + 8 * (i >> 2) + 4 * h + (i & 3);
    if (kr < L) {
      using G = typename std::conditional<GB, bf16, float>::type;
      G* dkr = static_cast<G*>(p.dk) + ((int64_t)(s0 + kr) * p.hkv + kvh) * DR;
      G* dvr = static_cast<G*>(p.dv) + ((int64_t)(s0 + kr) * p.hkv + kvh) * DR;
#pragma unroll
      for (int dt = 0; dt < DR / 32; ++dt) {
        dkr[32 * dt + lq] = (G)(st.dka[dt][i] * kmul);
        dvr[32 * dt + lq] = (G)st.dva[dt][i];
      }
    }
  }
}

// ------------------------------------------------- dK/dV, eight waves (D = 128)
//
// At D = 128 the four-wave kernel's K, V operands and dK, dV accumulators of
// 32 keys need ~360 registers, so each SIMD would run one wave with nothing
// to cover its latencies.  Here K and V of the 128-key tile stay in LDS and
// every 32-key slice gets two waves, one per 32-query half of each 64-query
// block: a wave holds its dK, dV accumulators (128 registers) and the scores
// of one half, fits 256 registers, and each SIMD runs two waves.  The price is
// LDS traffic: K and V are read again for every block (1.5 instead of 1 KB of
// operand reads per MFMA).  The two partial sums of a slice meet once per
// tile, through LDS.

constexpr int kThreads8 = 512;

template <int D>
struct DkvAcc {
  f32x16 dka[D / 32], dva[D / 32];
};

// One 64-query block for one wave of the eight-wave kernel: keys wk_lo .. +31
// (K, V rows at Kw, Vw in LDS) against the 32 queries qm .. qm + 31 (rows at
// Qh, dOh; their -lse / scale and -D at NLh, Dh):
//   A: S = Q K^T, dP = dO V^T - D   (16 MFMAs, row reads of all four operands)
//   B: P and dS in bf16, as the A operands of C (split in two 16-query slices)
//   C: dV += P^T dO, dK += dS^T Q    (16 MFMAs, column reads of dO and Q)
// The second slice of B runs between the MFMAs of C's first slice.
template <int D, bool MASK>
__device__ __forceinline__ void dkdv_half(DkvAcc<D>& st, const char* Qh, const char* dOh, const char* Kw,
                                          const char* Vw, const float* NLh, const float* Dh, float c2, int h,
                                          const TileReadOffsets& o, int32_t qm, int32_t key, int32_t L) {
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  // the accumulators start from -lse / scale and -D of the lane's query rows
  // (register i <-> query qm + 8 (i / 4) + 4 h + i % 4)
  f32x16 s, dp;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(NLh + 8 * g + 4 * h);
    const f32x4 v = *reinterpret_cast<const f32x4*>(Dh + 8 * g + 4 * h);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[4 * g + e] = a[e];
      dp[4 * g + e] = v[e];
    }
  }
  // A: both chains advance together, operands read PF k-steps ahead
  {
    constexpr int PF = 3;
    bf16x8 aq[KS], ak[KS], ad[KS], av[KS];
    auto rd = [&](int kk) {
      aq[kk] = ld8(Qh + row_off(o, kk));
      ak[kk] = ld8(Kw + row_off(o, kk));
      ad[kk] = ld8(dOh + row_off(o, kk));
      av[kk] = ld8(Vw + row_off(o, kk));
    };
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) rd(kk);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (kk + PF < KS) rd(kk + PF);
      s = mfma32(aq[kk], ak[kk], s);
      dp = mfma32(ad[kk], av[kk], dp);
    }
    PSC_SCHED_DS_READ(4 * PF + 4);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      PSC_SCHED_MFMA(2);
      if (kk + PF + 1 < KS) PSC_SCHED_DS_READ(4);
    }
  }
  // operands of C's first slice, read while A drains
  // (pair ks, dt covers queries 16 ks .. +15 and columns 32 dt .. +31)
  bf16x8 bo[DT], bq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    bo[dt] = col_operand(dOh, o, 0, dt);
    bq[dt] = col_operand(Qh, o, 0, dt);
  }
  if (MASK) mask_half(s, qm, key, L, h);
  bf16x8 pa[2], da[2];
  auto pds = [&](int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const float pr = fast_exp2(s[i] * c2);
      pa[i >> 3][i & 7] = (bf16)pr;
      da[i >> 3][i & 7] = (bf16)(pr * dp[i]);
    }
  };
  pds(0, 8);
  // C: first slice, with B's second slice and the second slice's operands
  // between its MFMAs
  bf16x8 bo1[DT], bq1[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    bo1[dt] = col_operand(dOh, o, 1, dt);
    bq1[dt] = col_operand(Qh, o, 1, dt);
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    st.dva[dt] = mfma32(pa[0], bo[dt], st.dva[dt]);
    st.dka[dt] = mfma32(da[0], bq[dt], st.dka[dt]);
  }
  pds(8, 16);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    st.dva[dt] = mfma32(pa[1], bo1[dt], st.dva[dt]);
    st.dka[dt] = mfma32(da[1], bq1[dt], st.dka[dt]);
  }
}

// Wave w takes keys kb + 32 (w % 4) .. +31 and the query half w / 4 of every
// block; the two waves of a key slice add their partial dK, dV at the end.
template <int D, bool GB = false, bool ROPE = false>
__global__ void __launch_bounds__(kThreads8, 1) k_bwd_dkdv8(BwdParams p) {
  constexpr int TB = tile_bytes<D>();
  constexpr int NW = kThreads8 / 64;
  constexpr int DT = D / 32;
  // Q, dO stage 0 | Q, dO stage 1 | K (2 tiles) | V (2 tiles) | lse, -D x 2:
  // the four stage tiles lie within the 64 KB that a ds_read offset field
  // reaches from one base, and so do K and V from another
  __shared__ __attribute__((aligned(16))) char sm[8 * TB + 4 * kBMk * sizeof(float)];
  char* const Qs0 = sm;
  char* const dOs0 = sm + TB;
  char* const Qs1 = sm + 2 * TB;
  char* const dOs1 = sm + 3 * TB;
  char* const Kt = sm + 4 * TB;
  char* const Vt = sm + 6 * TB;
  float* const NLs0 = reinterpret_cast<float*>(sm + 8 * TB);
  float* const Ds0 = NLs0 + kBMk;
  float* const NLs1 = Ds0 + kBMk;
  float* const Ds1 = NLs1 + kBMk;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, lq = l & 31;
  const int ks = w & 3, qh = w >> 2;
  const uint32_t item = blockIdx.x / (uint32_t)p.hkv, kvh = blockIdx.x % (uint32_t)p.hkv;
  // item < cap (the grid is cap work-groups per head), so the entry is read
  // together with the count and used only once the count admits it; every
  // entry below the count is written, with segment bounds clamped to [0, T].
  const int4 it = *reinterpret_cast<const int4*>(p.items + 4 * item);
  if ((int32_t)item >= *p.n_items) return;
  const int32_t s0 = it.x, L = it.y, tile = it.z;
  const int32_t kb = tile * kBKV;
  if (kb >= L) return;
  const int32_t wk_lo = kb + 32 * ks;
  const int32_t key = wk_lo + lq;  // this lane's key (S layout: lane <-> key)
  const int32_t nqb = (L - kb + kBMk - 1) / kBMk;
  const int32_t niter = p.group * nqb;

  uint32_t qoff[D / 8 / NW], ooff[D / 8 / NW];
  tile_offsets<D, NW>(p.sq, w, l, qoff);
  tile_offsets<D, NW>(p.sdo, w, l, ooff);
  {
    uint32_t koff[D / 8 / NW], voff[D / 8 / NW];
    tile_offsets<D, NW>(p.sk, w, l, koff);
    tile_offsets<D, NW>(p.sv, w, l, voff);
    const bf16* Kp = p.k + (int64_t)s0 * p.sk + (int64_t)kvh * D;
    const bf16* Vp = p.v + (int64_t)s0 * p.sv + (int64_t)kvh * D;
    load_tile<D, NW>(Kp, p.sk, kb, L, koff, Kt, w, l);
    load_tile<D, NW>(Kp, p.sk, kb + kTileRows, L, koff, Kt + TB, w, l);
    load_tile<D, NW>(Vp, p.sv, kb, L, voff, Vt, w, l);
    load_tile<D, NW>(Vp, p.sv, kb + kTileRows, L, voff, Vt + TB, w, l);
  }
  // iteration t: query head kvh*G + t / nqb, query block kb + (nqb - 1 - t % nqb) * 64,
  // from the document end back to the tile (as in the four-wave kernel)
  auto issue = [&](int32_t t, char* Qs, char* dOs, float* NLs, float* Ds) {
    const int32_t head = kvh * p.group + t / nqb;
    const int32_t qs = kb + (nqb - 1 - t % nqb) * kBMk;
    load_tile<D, NW>(p.q + (int64_t)s0 * p.sq + (int64_t)head * D, p.sq, qs, L, qoff, Qs, w, l);
    load_tile<D, NW>(p.dout + (int64_t)s0 * p.sdo + (int64_t)head * D, p.sdo, qs, L, ooff, dOs, w, l);
    if (w == 0) load_vec64_async(p.NLbuf + (int64_t)head * p.T + s0, qs, L, NLs, l);
    if (w == 1) load_vec64_async(p.Dbuf + (int64_t)head * p.T + s0, qs, L, Ds, l);
  };
  issue(0, Qs0, dOs0, NLs0, Ds0);

  DkvAcc<D> st;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    st.dka[dt] = f32x16{};
    st.dva[dt] = f32x16{};
  }
  const float c2 = p.scale_log2;
  const TileReadOffsets ro = tile_read_offsets(h, lq, l);
  // rows lq and 32 + lq share the swizzle, so a 32-row slice is a fixed offset
  const char* const Kw = Kt + (ks >> 1) * TB + (ks & 1) * 32 * 128;
  const char* const Vw = Vt + (ks >> 1) * TB + (ks & 1) * 32 * 128;
  auto block = [&](int32_t t, const char* Qs, const char* dOs, const float* NLs, const float* Ds) {
    const int32_t qm = kb + (nqb - 1 - t % nqb) * kBMk + 32 * qh;
    const char* Qh = Qs + qh * 32 * 128;
    const char* dOh = dOs + qh * 32 * 128;
    if (qm >= wk_lo + 31 && qm + 32 <= L)
      dkdv_half<D, false>(st, Qh, dOh, Kw, Vw, NLs + 32 * qh, Ds + 32 * qh, c2, h, ro, qm, key, L);
    else if (qm + 31 >= wk_lo && qm < L && wk_lo < L)
      dkdv_half<D, true>(st, Qh, dOh, Kw, Vw, NLs + 32 * qh, Ds + 32 * qh, c2, h, ro, qm, key, L);
  };
  for (int32_t t = 0; t < niter; t += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < niter) issue(t + 1, Qs1, dOs1, NLs1, Ds1);
    block(t, Qs0, dOs0, NLs0, Ds0);
    if (t + 1 >= niter) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 2 < niter) issue(t + 2, Qs0, dOs0, NLs0, Ds0);
    block(t + 1, Qs1, dOs1, NLs1, Ds1);
  }

  // The two waves of a key slice meet: the query-half-1 wave hands its dK over
  // and the half-0 wave its dV (regions of 16 KB, lane-major 16-byte pieces),
  // then each adds its partner's part to the one it keeps and stores it.
  __syncthreads();  // every wave is done with the tiles
  f32x4* const red = reinterpret_cast<f32x4*>(sm);
  constexpr int kPieces = DT * 4 * 64;  // f32x4 pieces per wave
  auto give = [&](const f32x16* x) {
    f32x4* mine = red + (2 * ks + qh) * kPieces;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        mine[(4 * dt + g) * 64 + l] = f32x4{x[dt][4 * g], x[dt][4 * g + 1], x[dt][4 * g + 2], x[dt][4 * g + 3]};
    }
  };
  // add the partner's part and store (C layout: key = wk_lo + 8*(i/4) + 4*h + i%4, d = 32*dt + lq)
  auto finish = [&](f32x16* x, void* outp, float mul, bool turn) {
    const f32x4* theirs = red + (2 * ks + (qh ^ 1)) * kPieces;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 y = theirs[(4 * dt + g) * 64 + l];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[dt][4 * g + e] += y[e];
      }
    }
    if constexpr (ROPE) {
      // dK of the turned k, scaled, turned back by -theta: dims d and d + D/2
      // of a key are x[dt] and x[dt + D/64] of the same lane and register
      if (turn) {
        constexpr int HD = D / 64;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int32_t kr = wk_lo + 8 * (i >> 2) + 4 * h + (i & 3);
          if (kr < L) {
            const float2* cs = rope_row(p, s0 + kr, D / 2);
#pragma unroll
            for (int dt = 0; dt < HD; ++dt) {
              const float2 t = cs[32 * dt + lq];
              float y1, y2;
              rope_turn(x[dt][i] * mul, x[dt + HD][i] * mul, t.x, -t.y, y1, y2);
              x[dt][i] = y1;
              x[dt + HD][i] = y2;
            }
          }
        }
        mul = 1.f;
      }
    } else {
      (void)turn;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int32_t kr = wk_lo + 8 * (i >> 2) + 4 * h + (i & 3);
      if (kr < L) {
        if constexpr (GB) {
          bf16* r = static_cast<bf16*>(outp) + ((int64_t)(s0 + kr) * p.hkv + kvh) * D;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) r[32 * dt + lq] = (bf16)(x[dt][i] * mul);
        } else {
          float* r = static_cast<float*>(outp) + ((int64_t)(s0 + kr) * p.hkv + kvh) * D;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) r[32 * dt + lq] = x[dt][i] * mul;
        }
      }
    }
  };
  if (qh) give(st.dka);
  else give(st.dva);
  __syncthreads();
  if (qh) finish(st.dva, p.dv, 1.f, false);
  else finish(st.dka, p.dk, p.scale, true);
}

}  // namespace

static size_t vec_bytes(const AttnDims& d) { return align_up(sizeof(float) * (size_t)d.hq * d.T, 256); }

// dQ kernel: query heads per workgroup, the largest of 4, 2, 1 that divides
// the group (its tiles are 128 / that rows high).
static int dq_heads_per_wg(const AttnDims& d) {
  const int g = d.hq / d.hkv;
  return g % 4 == 0 ? 4 : (g % 2 == 0 ? 2 : 1);
}

size_t attn_bwd_workspace_bytes(int dtype, const AttnDims& d) {
  if (dtype != 1) return vec_bytes(d);
  return 2 * vec_bytes(d) + schedule_bytes(d.T, d.n_seg, d.max_seqlen, kBQ / dq_heads_per_wg(d), kBNq) +
         schedule_bytes(d.T, d.n_seg, d.max_seqlen, kBKV, kBMk);
}

template <bool GB, bool ROPE>
static void launch_dq(int hd, int hp, unsigned grid, const BwdParams& p, hipStream_t stream) {
  if (hd == 128) {
    if (hp == 4) k_bwd_dq<128, 4, 128, GB, ROPE><<<grid, kThreads, 0, stream>>>(p);
    else if (hp == 2) k_bwd_dq<128, 2, 128, GB, ROPE><<<grid, kThreads, 0, stream>>>(p);
    else k_bwd_dq<128, 1, 128, GB, ROPE><<<grid, kThreads, 0, stream>>>(p);
  } else if (hd == 64) {
    if (hp == 4) k_bwd_dq<64, 4, 64, GB, ROPE><<<grid, kThreads, 0, stream>>>(p);
    else if (hp == 2) k_bwd_dq<64, 2, 64, GB, ROPE><<<grid, kThreads, 0, stream>>>(p);
    else k_bwd_dq<64, 1, 64, GB, ROPE><<<grid, kThreads, 0, stream>>>(p);
  } else if constexpr (!ROPE) {
    // head_dim 32: the D = 64 kernel on half-width heads
    if (hp == 4) k_bwd_dq<64, 4, 32, GB><<<grid, kThreads, 0, stream>>>(p);
    else if (hp == 2) k_bwd_dq<64, 2, 32, GB><<<grid, kThreads, 0, stream>>>(p);
    else k_bwd_dq<64, 1, 32, GB><<<grid, kThreads, 0, stream>>>(p);
  }
}

template <bool GB, bool ROPE>
static void launch_dkdv(int hd, unsigned grid, const BwdParams& p, hipStream_t stream) {
  if (hd == 128)
    k_bwd_dkdv8<128, GB, ROPE><<<grid, kThreads8, 0, stream>>>(p);
  else if (hd == 64)
    k_bwd_dkdv<64, 64, GB, ROPE><<<grid, kThreads, 0, stream>>>(p);
  else if constexpr (!ROPE)
    k_bwd_dkdv<64, 32, GB><<<grid, kThreads, 0, stream>>>(p);
}

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream) {
  const AttnDims& d = a.dims;
  char* ws = static_cast<char*>(a.workspace);
  float* Dbuf = reinterpret_cast<float*>(ws);
  ws += vec_bytes(d);
  float* NLbuf = reinterpret_cast<float*>(ws);
  ws += vec_bytes(d);
  const int hp = dq_heads_per_wg(d);
  TileSchedule sq = schedule_carve(ws, d.T, d.n_seg, d.max_seqlen, kBQ / hp, kBNq);
  ws += schedule_bytes(d.T, d.n_seg, d.max_seqlen, kBQ / hp, kBNq);
  TileSchedule sk = schedule_carve(ws, d.T, d.n_seg, d.max_seqlen, kBKV, kBMk);

  BwdParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.o = static_cast<const bf16*>(a.o);
  p.dout = static_cast<const bf16*>(a.dout);
  p.lse = a.lse;
  p.Dbuf = Dbuf;
  p.NLbuf = NLbuf;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.grad_bf16 = a.grad_bf16;
  p.pos = a.rope.pos;
  p.rope_cs = a.rope.rope_cs;
  p.rope_n_pos = a.rope.rope_n_pos;
  p.sq = a.sq;
  p.sk = a.sk;
  p.sv = a.sv;
  p.so = a.so;
  p.sdo = a.sdo;
  p.T = d.T;
  p.cu = a.cu;
  p.hq = d.hq;
  p.hkv = d.hkv;
  p.group = d.hq / d.hkv;
  p.scale = d.scale;
  p.scale_log2 = d.scale * kLog2e;
  if (d.T == 0) return hipSuccess;

  // dQ first: it also produces -D and -lse / scale, which dK/dV reads.
  hipError_t e = launch_schedule(a.cu, d.n_seg, (int32_t)d.T, kBQ / hp, kBNq, false, sq, stream);
  if (e != hipSuccess) return e;
  p.items = sq.items;
  p.n_items = sq.n_items;
  const unsigned grid_q = (unsigned)(sq.cap * (d.hq / hp));
  {
    ScopedKernelTimer timed(kTimeBwdDq, stream);
    if (p.rope_cs) {
      if (p.grad_bf16) launch_dq<true, true>(d.d, hp, grid_q, p, stream);
      else launch_dq<false, true>(d.d, hp, grid_q, p, stream);
    } else {
      if (p.grad_bf16) launch_dq<true, false>(d.d, hp, grid_q, p, stream);
      else launch_dq<false, false>(d.d, hp, grid_q, p, stream);
    }
  }

  e = launch_schedule(a.cu, d.n_seg, (int32_t)d.T, kBKV, kBMk, true, sk, stream);
  if (e != hipSuccess) return e;
  p.items = sk.items;
  p.n_items = sk.n_items;
  const unsigned grid_kv = (unsigned)(sk.cap * d.hkv);
  {
    ScopedKernelTimer timed(kTimeBwdDkdv, stream);
    if (p.rope_cs) {
      if (p.grad_bf16) launch_dkdv<true, true>(d.d, grid_kv, p, stream);
      else launch_dkdv<false, true>(d.d, grid_kv, p, stream);
    } else {
      if (p.grad_bf16) launch_dkdv<true, false>(d.d, grid_kv, p, stream);
      else launch_dkdv<false, false>(d.d, grid_kv, p, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace psc
