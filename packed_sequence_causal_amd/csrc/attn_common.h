// Device primitives shared by the bf16 attention kernels (gfx950 / CDNA4).
//
// MFMA operand layouts (v_mfma_f32_32x32x16_bf16, one 64-lane wave):
//   A (32 x 16, M x K): lane l holds A[l % 32][8*(l/32) + j], j = 0..7
//   B (16 x 32, K x N): lane l holds B[8*(l/32) + j][l % 32]
//   C (32 x 32):        lane l, register i holds C[8*(i/4) + 4*(l/32) + i%4][l % 32]
// The kernels keep one query (or one key) per lane in the C layout and treat
// the sixteen C registers of a 32-row tile as two k-steps of the next product:
// k-slot (half h = l/32, j) of k-step s stands for row 16*s + kperm(h, j) with
//   kperm(h, j) = 8*(j/4) + 4*h + j%4.
// Any permutation of a contraction index is allowed as long as both operands
// use it, so the second operand is read from LDS in the same order.
//
// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i%4 of the four-element vectors addressed by lanes 4*j + i/4 (j = 0..3).
// With lane L of the group pointing at &M[r0 + L/4][c0 + 4*(L%4)] of a
// row-major matrix M, lane i receives M[r0 + j][c0 + i] for j = 0..3: a column
// read of four consecutive rows.  Two such reads fill one 8-element operand.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace psc {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define PSC_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two transposing LDS reads: rows r0..r0+3 and r0+8..r0+11 of column
// c0 + (lane % 16), as laid out for k-slots kperm(h, 0..7) with r0 = base + 4*h.
// `p0`/`p1` are the per-lane addresses already offset for the lane (see
// tr_addr below).
__device__ __forceinline__ bf16x8 tr_read8(const bf16* p0, const bf16* p1) {
  s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PSC_LDS s16x4*)(p0));
  s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PSC_LDS s16x4*)(p1));
  bf16x4 x = __builtin_bit_cast(bf16x4, a);
  bf16x4 y = __builtin_bit_cast(bf16x4, b);
  return bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// Partner value across the two 32-lane halves of the wave (lane l <-> l ^ 32).
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Map a hardware workgroup id to a logical one so that `g` consecutive logical
// ids (the query heads that share one key/value head) run on the same XCD.
// Workgroups are dispatched round-robin over the 8 XCDs; the last partial
// window keeps the identity map.
__device__ __forceinline__ uint32_t xcd_group_remap(uint32_t b, uint32_t n, uint32_t g) {
  if (g <= 1) return b;
  const uint32_t win = 8u * g;
  const uint32_t c = b / win;
  if ((c + 1) * win > n) return b;
  const uint32_t r = b - c * win;
  return c * win + (r % 8u) * g + r / 8u;
}

// Asynchronous global -> LDS copy of 16 (or 4) bytes per lane:
// global_load_lds_dwordx4 writes lane i's data to LDS byte M0 + 16*i.  Issued
// through inline assembly so the compiler's wait-count bookkeeping does not
// see it: once such a copy is in flight LLVM can only wait for *all*
// outstanding LDS reads (lgkmcnt(0)) instead of the ones an MFMA needs.
// Completion is the caller's job: s_waitcnt vmcnt(0) then a barrier before
// the destination is read, and no read of a destination while it is written.
// `lds` must be wave-uniform.  An LDS-DMA load may read M0 only one wait
// state after a scalar instruction wrote it, hence the s_nop 0.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src)
               : "memory", "m0");
}
// lds_dma16 with a uniform 64-bit base (SGPRs) and a 32-bit per-lane byte
// offset: the address needs no per-lane arithmetic.  The base often comes
// from v_readfirstlane just before the statement, and a vector memory
// instruction may read an SGPR only 5 wait states after a VALU wrote it; the
// compiler cannot see inside the asm, so the wait states are in it (s_nop 2,
// the m0 move and the s_nop 0 that M0 needs).
__device__ __forceinline__ void lds_dma16_sv(const void* sbase, uint32_t voff, uint32_t lds) {
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  const uint64_t b = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  asm volatile("s_nop 2\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff),
               "s"(b)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(src)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((PSC_LDS const char*)p);
}

// ------------------------------------------------------------------ LDS tiles
//
// A tile of 64 rows x D bf16 columns is stored as D/64 column groups of eight
// 16-byte chunks (128 bytes of each row); inside a group the rows are 128
// bytes apart and chunk j of row r sits in slot j ^ swz(r).  swz was chosen
// (checked exhaustively for 64 four-byte banks) so that both read patterns of
// the kernels are free of bank conflicts:
//   * MFMA operand rows (ds_read_b128): 16 lanes read chunk c of 16
//     consecutive rows;
//   * column reads (ds_read_b64_tr_b16): a 16-lane group reads 8-byte halves
//     of chunks c and c+1 (c even) of 4 consecutive rows starting at a
//     multiple of 4;
// and, since swz(r) depends only on bits 1..3 of r, a lane needs just a few
// precomputed offsets for all its reads.  One asynchronous load instruction
// fills 8 rows of one group: 8 contiguous 128-byte row pieces from global
// memory.
constexpr int kTileRows = 64;
constexpr int kGroupBytes = kTileRows * 128;
template <int D>
constexpr int tile_bytes() { return (D / 64) * kGroupBytes; }

__device__ __forceinline__ int lds_swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// Byte offset of element e (a multiple of 4) of row r.
__device__ __forceinline__ int lds_byte(int r, int e) {
  const int c = e >> 3;
  return (c >> 3) * kGroupBytes + r * 128 + (((c & 7) ^ lds_swz(r)) << 4) + (e & 7) * 2;
}

// Asynchronous load of rows [row0, row0 + 64) of a [T, heads, D] operand (base
// already points at the segment start and head) into one LDS tile, spread
// over NW waves (w = this wave).  global_load_lds_dwordx4 writes the 64 lanes'
// 16 bytes to 64 consecutive LDS slots; instruction t covers rows
// 8*(t%8) .. +7 of column group t/8, and each lane fetches the chunk that the
// swizzle places at its slot.  Rows at or past `L` repeat row L - 1: their
// scores are masked, any finite data will do.  Completion is tracked by
// vmcnt; wait, then barrier, before reading the tile.
// DR < D (a head of DR = D/2 columns held in a D-column tile): chunk c of a
// row is fetched from chunk c mod DR/8, so the columns past the head repeat
// its first ones; the kernels zero those columns of their register operand
// (scores are unchanged) or drop the results that read them.
template <int D, int NW, int DR = D>
__device__ __forceinline__ void load_tile_async(const bf16* base, int64_t stride, int32_t row0, int32_t L,
                                                void* lds, int w, int l) {
  constexpr int LOADS = D / 8;  // 64 rows x D/8 chunks / 64 lanes
  static_assert(LOADS % NW == 0, "tile loads must split evenly over the waves");
  const int rr = l >> 3;   // row inside the 8-row piece
  const int p = l & 7;     // slot inside the row
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t lds0 = lds_addr(lds);
#pragma unroll
  for (int i = 0; i < LOADS / NW; ++i) {
    const int t = w + NW * i;
    const int tu = wu + NW * i;
    const int g = t >> 3;
    const int r = 8 * (t & 7) + rr;
    const int c0 = 8 * g + (p ^ lds_swz(r));
    const int c = DR == D ? c0 : c0 % (DR / 8);
    const bf16* src = base + (int64_t)min(row0 + r, L - 1) * stride + c * 8;
    lds_dma16(src, lds0 + (tu >> 3) * kGroupBytes + (tu & 7) * 1024);
  }
}

// Per-lane byte offsets (from the tile's first row) of the chunks this wave
// fetches in load_tile_async, for a tile that needs no row clamping.
// stride * 128 must stay below 2^32 (checked by the host API).
template <int D, int NW, int DR = D>
__device__ __forceinline__ void tile_offsets(int64_t stride, int w, int l, uint32_t* off) {
  constexpr int LOADS = D / 8;
  const int rr = l >> 3;
  const int p = l & 7;
#pragma unroll
  for (int i = 0; i < LOADS / NW; ++i) {
    const int t = w + NW * i;
    const int g = t >> 3;
    const int r = 8 * (t & 7) + rr;
    const int c0 = 8 * g + (p ^ lds_swz(r));
    const int c = DR == D ? c0 : c0 % (DR / 8);
    off[i] = (uint32_t)(((int64_t)r * stride + c * 8) * 2);
  }
}

// load_tile_async for rows [row0, row0 + 64) all inside the segment; `rows`
// points at row row0 (wave-uniform), `off` from tile_offsets.
template <int D, int NW>
__device__ __forceinline__ void load_tile_async_full(const bf16* rows, const uint32_t* off, void* lds, int w) {
  constexpr int LOADS = D / 8;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t lds0 = lds_addr(lds);
#pragma unroll
  for (int i = 0; i < LOADS / NW; ++i) {
    const int tu = wu + NW * i;
    lds_dma16_sv(rows, off[i], lds0 + (tu >> 3) * kGroupBytes + (tu & 7) * 1024);
  }
}

// load_tile_async with the offset-only fast path for tiles inside the
// segment (`off` from tile_offsets<D, NW, DR> for this stride).
template <int D, int NW, int DR = D>
__device__ __forceinline__ void load_tile(const bf16* base, int64_t stride, int32_t row0, int32_t L,
                                          const uint32_t* off, void* lds, int w, int l) {
  if (row0 + kTileRows <= L)
    load_tile_async_full<D, NW>(base + (int64_t)row0 * stride, off, lds, w);
  else
    load_tile_async<D, NW, DR>(base, stride, row0, L, lds, w, l);
}

// Asynchronous load of 64 consecutive floats vec[row0 .. row0 + 64) (rows at or
// past L repeat row L - 1) into LDS, one 4-byte slot per lane of one wave.
__device__ __forceinline__ void load_vec64_async(const float* vec, int32_t row0, int32_t L, void* lds, int l) {
  const int32_t row = min(row0 + l, L - 1);
  lds_dma4(vec + row, lds_addr(lds));
}

// Scheduling hints: keep `n` LDS reads / MFMAs / VALU ops together, in the
// order the calls appear (llvm.amdgcn.sched.group.barrier masks).
#define PSC_SCHED_DS_READ(n) __builtin_amdgcn_sched_group_barrier(0x0100, (n), 0)
#define PSC_SCHED_MFMA(n) __builtin_amdgcn_sched_group_barrier(0x0008, (n), 0)
#define PSC_SCHED_VALU(n) __builtin_amdgcn_sched_group_barrier(0x0002, (n), 0)

// Per-lane LDS byte offsets of the two operand read patterns in a tile.  The
// swizzle depends on row bits 1..3 only, so moving 16 rows down or one column
// group right is a constant, and a few per-lane bases cover every read; the
// constants go into the instructions' offset fields instead of registers.
//   row[k]:    row lq, columns 16k + 8h (k = 0..3) -- the 16-byte MFMA
//              operand of k-step k; +kGroupBytes per 4 k-steps, +32*128 for
//              rows 32 + lq
//   col[e][u]: column read (ds_read_b64_tr_b16) of rows 4h + gi/4 + 8u and
//              columns 32e + dsub + 4 (gi % 4), gi = lane % 16, dsub =
//              16 ((lane / 16) % 2); +2048 per 16 rows, +kGroupBytes per 64
//              columns
struct TileReadOffsets {
  uint32_t row[4];
  uint32_t col[2][2];
};

__device__ __forceinline__ TileReadOffsets tile_read_offsets(int h, int lq, int l) {
  TileReadOffsets o;
#pragma unroll
  for (int k = 0; k < 4; ++k) o.row[k] = (uint32_t)lds_byte(lq, 16 * k + 8 * h);
  const int gi = l & 15;
  const int dsub = 16 * ((l >> 4) & 1);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      o.col[e][u] = (uint32_t)lds_byte(4 * h + (gi >> 2) + 8 * u, 32 * e + dsub + 4 * (gi & 3));
  }
  return o;
}
// Offset of the row operand of k-step kk (lds_byte(lq, 16 kk + 8 h)).
__device__ __forceinline__ uint32_t row_off(const TileReadOffsets& o, int kk) {
  return o.row[kk & 3] + (kk >> 2) * kGroupBytes;
}
// Offset of column read u of 16-row slice ks and 32-column slice dt
// (lds_byte(16 ks + 4 h + gi/4 + 8 u, 32 dt + dsub + 4 (gi % 4))).
__device__ __forceinline__ uint32_t col_off(const TileReadOffsets& o, int u, int ks, int dt) {
  return o.col[dt & 1][u] + ks * 2048 + (dt >> 1) * kGroupBytes;
}
// Column-read operand (two transposing reads) of slice (ks, dt) at tile M.
__device__ __forceinline__ bf16x8 col_operand(const char* M, const TileReadOffsets& o, int ks, int dt) {
  return tr_read8(reinterpret_cast<const bf16*>(M + col_off(o, 0, ks, dt)),
                  reinterpret_cast<const bf16*>(M + col_off(o, 1, ks, dt)));
}

// acc[n] += A_n B over k = 0..KS-1 for two row blocks n = 0, 1 whose A
// fragments are 16-byte LDS reads at a0 + off(kk) and a1 + off(kk), with one
// k-step of read-ahead so every MFMA finds its operands already loaded.
template <int KS, typename Off>
__device__ __forceinline__ void mfma_rows2(f32x16& acc0, f32x16& acc1, const char* a0, const char* a1,
                                           const bf16x8* b, Off off) {
  bf16x8 x0 = *reinterpret_cast<const bf16x8*>(a0 + off(0));
  bf16x8 x1 = *reinterpret_cast<const bf16x8*>(a1 + off(0));
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    bf16x8 y0 = x0, y1 = x1;
    if (kk + 1 < KS) {
      x0 = *reinterpret_cast<const bf16x8*>(a0 + off(kk + 1));
      x1 = *reinterpret_cast<const bf16x8*>(a1 + off(kk + 1));
    }
    acc0 = mfma32(y0, b[kk], acc0);
    acc1 = mfma32(y1, b[kk], acc1);
  }
  PSC_SCHED_DS_READ(2);
#pragma unroll
  for (int kk = 0; kk + 1 < KS; ++kk) {
    PSC_SCHED_DS_READ(2);
    PSC_SCHED_MFMA(2);
  }
  PSC_SCHED_MFMA(2);
}

// acc += A B over k = 0..KS-1 for one row block (mfma_rows2 with a single
// accumulator), one k-step of read-ahead.
template <int KS, typename Off>
__device__ __forceinline__ void mfma_rows1(f32x16& acc, const char* a0, const bf16x8* b, Off off) {
  bf16x8 x0 = *reinterpret_cast<const bf16x8*>(a0 + off(0));
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    bf16x8 y0 = x0;
    if (kk + 1 < KS) x0 = *reinterpret_cast<const bf16x8*>(a0 + off(kk + 1));
    acc = mfma32(y0, b[kk], acc);
  }
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace psc
