// Document-causal attention forward, bf16 in / fp32 accumulate, gfx950.
//
// One workgroup = one query tile inside one document for HP query heads of
// one key/value group (HP = 4, 2 or 1, the largest dividing the group): the
// tile is 128 / HP rows high and each of the four waves owns 32 rows of one
// head, so with HP = 4 the waves share rows and key/value blocks and do
// equal work.  The key/value loop runs over
// 64-key blocks from the document start to the tile's last row, so only tiles
// inside the document's causal triangle are visited and no mask is stored
// ("Sample Packing：长序列 LLM 训练的 Attention 问题及优化", sections 三 and 5.1).
//
// Key/value blocks are double-buffered in LDS and filled with asynchronous
// direct-to-LDS loads (global_load_lds_dwordx4): block j+1 streams in while
// block j is computed, and no VGPR holds staging data.  Because each load
// instruction writes 64 consecutive 16-byte LDS slots in lane order, the tile
// layout is chosen by which global chunk each lane fetches: chunk c of row r
// sits in slot c ^ swz(r) of that row (see lds_slot), which keeps both the
// row reads of K and the column reads of V free of bank conflicts.
//
// Per 64-key block and wave (layouts in attn_common.h):
//   S^T = K Q^T    A = K rows from LDS, B = Q kept in registers; each lane
//                  then holds 32 scores of its own query row.
//   online softmax in the exp2 domain: raw-score max, one fma + exp2 per
//                  score, and the running max is raised only when a row's max
//                  grows by more than 2^8 (so O and l are rescaled rarely; the
//                  result is exact either way, p just stays below 2^8).
//   O^T += V^T P^T A = V read column-wise from LDS with ds_read_b64_tr_b16,
//                  B = P rounded to bf16 straight from the score registers.
// Epilogue: O / l in bf16, lse = (m + log2 l) * ln 2 in fp32.
#include "attn_common.h"
#include "psc_internal.h"
#include "rope_common.h"

namespace psc {
namespace {

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per block
constexpr int kThreads = 256;
constexpr float kRescaleSlack = 8.0f;  // log2 units

struct FwdParams {
  const bf16 *q, *k, *v;
  bf16* out;
  float* lse;
  int64_t sq, sk, sv, so, T;
  const int32_t* cu;
  const int32_t* items;
  const int32_t* n_items;
  int32_t hq, group;
  float scale_log2;
  // rotary embedding of q inside the kernel (the ROPE instantiations only)
  bf16* q_rot;             // q turned, written in place
  const int32_t* pos;      // [T] position of each token
  const float2* rope_cs;   // [rope_n_pos][D/2] (cos, sin)
  int32_t rope_n_pos;
};

// Asynchronous loads of key/value rows [kb, kb + 64) into one LDS stage.
template <int D, int DR>
__device__ __forceinline__ void load_kv(const bf16* Kp, const bf16* Vp, int64_t sk, int64_t sv, int32_t kb,
                                        int32_t L, char* Ks, char* Vs, const uint32_t* koff, const uint32_t* voff,
                                        int w, int l) {
  load_tile<D, kThreads / 64, DR>(Kp, sk, kb, L, koff, Ks, w, l);
  load_tile<D, kThreads / 64, DR>(Vp, sv, kb, L, voff, Vs, w, l);
}

template <int D>
struct FwdState {
  bf16x8 qf[D / 16];
  f32x16 oacc[D / 32];
  float m_i, l_i;
};

// One 64-key block for one wave.
template <int D>
__device__ __forceinline__ void fwd_block(FwdState<D>& st, const char* Ks, const char* Vs, int32_t kb, int32_t L,
                                          int32_t qrow, int32_t wq_lo, float c2, int h, const TileReadOffsets& o) {
  const char* Kb = reinterpret_cast<const char*>(Ks);
  const char* Vb = reinterpret_cast<const char*>(Vs);
  f32x16 s[2] = {f32x16{}, f32x16{}};
  // rows lq and 32 + lq share the swizzle (it depends on row bits 1..3 only)
  mfma_rows2<D / 16>(s[0], s[1], Kb, Kb + 32 * 128, st.qf, [&](int kk) { return row_off(o, kk); });
  if ((kb + kBN - 1 > wq_lo) || (kb + kBN > L)) {
    // key kb + 32 n2 + 8 (i / 4) + 4 h + i % 4 is masked when it is after the
    // row or at/after the document end: one compare with a constant per score
    const int32_t lim = min(qrow + 1, L) - kb - 4 * h;
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (32 * n2 + 8 * (i >> 2) + (i & 3) >= lim) s[n2][i] = -INFINITY;
      }
    }
  }
  float mx = s[0][0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
  mx = max_halves(mx) * c2;
  // raise the running max only when this block's max exceeds it by > 2^8
  if (__builtin_amdgcn_ballot_w64(mx > st.m_i + kRescaleSlack) != 0) {
    const float m_new = fmaxf(st.m_i, mx);
    const float alpha = fast_exp2(st.m_i - m_new);
    st.l_i *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) st.oacc[dt] *= alpha;
    st.m_i = m_new;
  }
  const float neg_m = -st.m_i;
  float rs = 0.f;
  bf16x8 pb[4];
#pragma unroll
  for (int n2 = 0; n2 < 2; ++n2) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = fast_exp2(__builtin_fmaf(s[n2][i], c2, neg_m));
      rs += e;
      pb[2 * n2 + (i >> 3)][i & 7] = (bf16)e;
    }
  }
  st.l_i += rs;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) st.oacc[dt] = mfma32(col_operand(Vb, o, ks, dt), pb[ks], st.oacc[dt]);
  }
}

// HP query heads of one key/value group per workgroup (1, 2 or 4), each on
// 128 / HP rows: wave w takes head w % HP and rows 32 (w / HP) .. +31 of the
// tile, so with HP = 4 all four waves cover the same rows (equal work) and
// share every key/value block.
// DR = D / 2 runs heads of DR columns in the D-column kernel: Q's columns past
// DR are zero in registers (so the scores are those of the DR columns), the
// tile loader repeats the head's columns there, and only O's first DR
// columns are stored.
// ROPE: Q's rows are turned by their tokens' positions as they are loaded
// (rope_common.h; K arrives already turned) and written back in place, so the
// backward reads the turned q.  Each (row, head) of q belongs to one
// workgroup, which reads it before writing it.
template <int D, int HP, int DR = D, bool ROPE = false>
__global__ void __launch_bounds__(kThreads, 2) k_attn_fwd(FwdParams p) {
  static_assert(DR == D || 2 * DR == D, "a head fills the tile or half of it");
  constexpr int RW = kBM / HP;  // query rows per workgroup
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
  // item < cap (the grid is cap work-groups per head), so the entry is read
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

  const bf16* Qp = p.q + (int64_t)s0 * p.sq + (int64_t)head * DR;
  const bf16* Kp = p.k + (int64_t)s0 * p.sk + (int64_t)kvh * DR;
  const bf16* Vp = p.v + (int64_t)s0 * p.sv + (int64_t)kvh * DR;

  const int32_t kv_end = min(q0 + RW, L);
  const int32_t nkv = (kv_end + kBN - 1) / kBN;
  uint32_t koff[D / 8 / (kThreads / 64)], voff[D / 8 / (kThreads / 64)];
  tile_offsets<D, kThreads / 64, DR>(p.sk, w, l, koff);
  tile_offsets<D, kThreads / 64, DR>(p.sv, w, l, voff);
  load_kv<D, DR>(Kp, Vp, p.sk, p.sv, 0, L, Ks0, Vs0, koff, voff, w, l);

  const int32_t qrow = q0 + 32 * rs + lq;
  const bool qvalid = qrow < L;
  FwdState<D> st;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    st.qf[kk] = qvalid && 16 * kk + 8 * h < DR
                    ? *reinterpret_cast<const bf16x8*>(Qp + (int64_t)qrow * p.sq + 16 * kk + 8 * h)
                    : bf16x8{};
  }
  if constexpr (ROPE) {
    // dims i and i + DR/2 of the lane's row sit in k-steps kk and kk + DR/32
    // (element j) of the same lane
    static_assert(DR == D, "the turn pairs k-steps of one lane");
    constexpr int HK = DR / 32;
    if (qvalid) {
      const int32_t pos = min(max(p.pos[s0 + qrow], 0), p.rope_n_pos - 1);
      const float2* cs = p.rope_cs + (int64_t)pos * (DR / 2) + 8 * h;
#pragma unroll
      for (int kk = 0; kk < HK; ++kk) {
        float4 t4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t4[u] = reinterpret_cast<const float4*>(cs + 16 * kk)[u];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float c = (j & 1) ? t4[j >> 1].z : t4[j >> 1].x;
          const float sn = (j & 1) ? t4[j >> 1].w : t4[j >> 1].y;
          float y1, y2;
          rope_turn((float)st.qf[kk][j], (float)st.qf[kk + HK][j], c, sn, y1, y2);
          st.qf[kk][j] = (bf16)y1;
          st.qf[kk + HK][j] = (bf16)y2;
        }
      }
      bf16* Qw = p.q_rot + (int64_t)(s0 + qrow) * p.sq + (int64_t)head * DR;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) *reinterpret_cast<bf16x8*>(Qw + 16 * kk + 8 * h) = st.qf[kk];
    }
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.oacc[dt] = f32x16{};
  st.m_i = -INFINITY;
  st.l_i = 0.f;

  const int32_t wq_lo = q0 + 32 * rs, wq_hi = wq_lo + 31;
  // last key block a wave needs: up to its last row; none when all its rows
  // are past the document end (the tile's ragged tail)
  const int32_t wq_top = wq_lo < L ? wq_hi : -1;
  const float c2 = p.scale_log2;
  const TileReadOffsets ro = tile_read_offsets(h, lq, l);
  for (int32_t j = 0; j < nkv; j += 2) {
    // stage 0 holds block j
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < nkv) load_kv<D, DR>(Kp, Vp, p.sk, p.sv, (j + 1) * kBN, L, Ks1, Vs1, koff, voff, w, l);
    if (j * kBN <= wq_top) fwd_block<D>(st, Ks0, Vs0, j * kBN, L, qrow, wq_lo, c2, h, ro);
    if (j + 1 >= nkv) break;
    // stage 1 holds block j + 1
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 2 < nkv) load_kv<D, DR>(Kp, Vp, p.sk, p.sv, (j + 2) * kBN, L, Ks0, Vs0, koff, voff, w, l);
    if ((j + 1) * kBN <= wq_top) fwd_block<D>(st, Ks1, Vs1, (j + 1) * kBN, L, qrow, wq_lo, c2, h, ro);
  }

  // Epilogue.  O goes out through LDS so that each store instruction writes
  // whole 2*D-byte rows (64 lanes x 16 bytes) instead of 16-byte pieces of
  // 32 rows: the stage the last block did not use is free (its block was
  // consumed before the last barrier, and no load targets it), and each wave
  // stages its 32 rows in its own half of one of its two tiles.  Inside a
  // row, 16-byte chunk c sits at slot c ^ (row % (D/8)).
  const float lt = sum_halves(st.l_i);
  const float inv = qvalid ? 1.f / lt : 0.f;
  {
    constexpr int kChunks = D / 8;
    char* stage = (nkv & 1) ? (w < 2 ? Ks1 : Vs1) : (w < 2 ? Ks0 : Vs0);
    char* ob = stage + (w & 1) * (tile_bytes<D>() / 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (bf16)(st.oacc[dt][4 * g4 + e] * inv);
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
      if (row < L && 8 * c < DR)
        *reinterpret_cast<bf16x8*>(p.out + (int64_t)(s0 + row) * p.so + (int64_t)head * DR + 8 * c) = v8;
    }
  }
  if (qvalid && h == 0) p.lse[(int64_t)head * p.T + s0 + qrow] = (st.m_i + __log2f(lt)) * kLn2;
}

}  // namespace

// Query heads per workgroup: the largest of 4, 2, 1 that divides the group.
static int heads_per_wg(const AttnDims& d) {
  const int g = d.hq / d.hkv;
  return g % 4 == 0 ? 4 : (g % 2 == 0 ? 2 : 1);
}

size_t attn_fwd_workspace_bytes(int dtype, const AttnDims& d) {
  if (dtype != 1) return 256;
  return schedule_bytes(d.T, d.n_seg, d.max_seqlen, kBM / heads_per_wg(d), kBN);
}

template <bool ROPE>
static void launch_fwd(int hd, int hp, unsigned g, const FwdParams& p, hipStream_t stream) {
  if (hd == 128) {
    if (hp == 4) k_attn_fwd<128, 4, 128, ROPE><<<g, kThreads, 0, stream>>>(p);
    else if (hp == 2) k_attn_fwd<128, 2, 128, ROPE><<<g, kThreads, 0, stream>>>(p);
    else k_attn_fwd<128, 1, 128, ROPE><<<g, kThreads, 0, stream>>>(p);
  } else if (hd == 64) {
    if (hp == 4) k_attn_fwd<64, 4, 64, ROPE><<<g, kThreads, 0, stream>>>(p);
    else if (hp == 2) k_attn_fwd<64, 2, 64, ROPE><<<g, kThreads, 0, stream>>>(p);
    else k_attn_fwd<64, 1, 64, ROPE><<<g, kThreads, 0, stream>>>(p);
  } else if constexpr (!ROPE) {
    // head_dim 32: the D = 64 kernel on half-width heads (no in-kernel turn)
    if (hp == 4) k_attn_fwd<64, 4, 32><<<g, kThreads, 0, stream>>>(p);
    else if (hp == 2) k_attn_fwd<64, 2, 32><<<g, kThreads, 0, stream>>>(p);
    else k_attn_fwd<64, 1, 32><<<g, kThreads, 0, stream>>>(p);
  }
}

hipError_t launch_attn_fwd_bf16(const AttnFwdArgs& a, hipStream_t stream) {
  const AttnDims& d = a.dims;
  const int hp = heads_per_wg(d);
  TileSchedule s = schedule_carve(a.workspace, d.T, d.n_seg, d.max_seqlen, kBM / hp, kBN);
  hipError_t e = launch_schedule(a.cu, d.n_seg, (int32_t)d.T, kBM / hp, kBN, false, s, stream);
  if (e != hipSuccess) return e;
  FwdParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.out = static_cast<bf16*>(a.out);
  p.lse = a.lse;
  p.sq = a.sq;
  p.sk = a.sk;
  p.sv = a.sv;
  p.so = a.so;
  p.T = d.T;
  p.cu = a.cu;
  p.items = s.items;
  p.n_items = s.n_items;
  p.hq = d.hq;
  p.group = d.hq / d.hkv;
  p.scale_log2 = d.scale * kLog2e;
  const uint64_t grid = (uint64_t)s.cap * (uint64_t)d.hq;
  if (grid == 0) return hipSuccess;
  ScopedKernelTimer timed(kTimeFwd, stream);
  const unsigned g = (unsigned)(grid / hp);
  if (a.rope.rope_cs) {
    p.q_rot = static_cast<bf16*>(const_cast<void*>(a.q));
    p.pos = a.rope.pos;
    p.rope_cs = a.rope.rope_cs;
    p.rope_n_pos = a.rope.rope_n_pos;
    launch_fwd<true>(d.d, hp, g, p, stream);
  } else {
    launch_fwd<false>(d.d, hp, g, p, stream);
  }
  return hipGetLastError();
}

}  // namespace psc
