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

// ------------------------------------------------------------------ LDS tiles
//
// A tile of ROWS rows x D bf16 columns lives in LDS without padding, as 16-byte
// chunks; chunk c of row r sits in slot c ^ swz(r) of that row.  The swizzle
// keeps the two read patterns the kernels use free of bank conflicts: 16 lanes
// reading chunk c of 16 consecutive rows (MFMA operand rows, ds_read_b128),
// and ds_read_b64_tr_b16 groups reading 8-byte pieces of chunks c, c+1 (c
// even) of 4 consecutive rows starting at a multiple of 4.
template <int D>
__device__ __forceinline__ int lds_slot(int r, int c) {
  if constexpr (D == 128) return c ^ (((r & 7) << 1) | ((r >> 3) & 1));
  else return c ^ (((r & 3) << 1) | ((r >> 2) & 1));
}
// Byte offset of element e (a multiple of 4) of row r.
template <int D>
__device__ __forceinline__ int lds_byte(int r, int e) {
  return (r * (D / 8) + lds_slot<D>(r, e >> 3)) * 16 + (e & 7) * 2;
}

// Asynchronous load of rows [row0, row0 + ROWS) of a [T, heads, D] operand
// (base already points at the segment start and head) into one LDS tile,
// spread over NW waves (w = this wave).  global_load_lds_dwordx4 writes 64
// consecutive 16-byte slots in lane order, so each lane fetches the global
// chunk that belongs at its slot (the swizzle is an involution).  Rows at or
// past `L` repeat row L - 1: their scores are masked, any finite data will do.
// Completion is tracked by vmcnt; wait, then barrier, before reading the tile.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void load_tile_async(const bf16* base, int64_t stride, int32_t row0, int32_t L,
                                                void* lds, int w, int l) {
  constexpr int CPR = D / 8;
  constexpr int LOADS = ROWS * CPR / 64;
  static_assert(LOADS % NW == 0, "tile loads must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < LOADS / NW; ++i) {
    const int t = w + NW * i;
    const int slot = 64 * t + l;
    const int r = slot / CPR;
    const int c = lds_slot<D>(r, slot % CPR);
    const int32_t row = min(row0 + r, L - 1);
    __builtin_amdgcn_global_load_lds(base + (int64_t)row * stride + c * 8,
                                     (PSC_LDS void*)(static_cast<char*>(lds) + 64 * t * 16), 16, 0, 0);
  }
}

// Asynchronous load of 64 consecutive floats vec[row0 .. row0 + 64) (rows at or
// past L repeat row L - 1) into LDS, one 4-byte slot per lane of one wave.
__device__ __forceinline__ void load_vec64_async(const float* vec, int32_t row0, int32_t L, void* lds, int l) {
  const int32_t row = min(row0 + l, L - 1);
  __builtin_amdgcn_global_load_lds(vec + row, (PSC_LDS void*)lds, 4, 0, 0);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace psc
