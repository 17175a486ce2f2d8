// LDS tile layout and MFMA operand fetches shared by the MFMA kernels.
//
// Tiles of 16-bit elements are stored row-major with rows of D elements and
// no padding.  The 16-byte chunk c of row r lives at chunk position
// c ^ swz(r), where swz is linear (over GF(2)) in the low four bits of r.
// The weights were chosen so that both ways the kernels read a tile are free
// of bank conflicts, whether the LDS serves 128 or 256 bytes per clock:
//
//  * row reads (ds_read_b128): lane l reads 8 consecutive elements of row
//    (base + l%32), the operand layout of a 32x32x16 MFMA whose M or N index
//    runs along the tile's rows;
//  * transposed reads (ds_read_b64_tr_b16): each 16-lane group names four
//    rows times four 8-byte column groups; the instruction hands lane i of the
//    group element i%4 of the chunks named by lanes 4e + i/4 (e = 0..3), i.e.
//    four consecutive rows of one column.  Two such reads give an MFMA operand
//    whose contraction index runs along the tile's rows.
//
// Contraction slot order.  A 32x32 accumulator holds, in register r of lane l,
// row 8*(r/4) + 4*(l/32) + r%4.  When those accumulators (rounded to 16 bits)
// become the operand of the next product, slot s (0..7) of lane group
// g = l/32 in 16-row chunk c stands for row 16c + 8*(s/4) + 4g + s%4.  The
// transposed reads below fetch exactly that order.
#pragma once

#include <type_traits>

#include "fa_common.h"

namespace fa {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
  static __device__ __forceinline__ f32x16 mac(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<_Float16> {
  static __device__ __forceinline__ f32x16 mac(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

// Chunk swizzle of row r.
template <int D> __device__ __forceinline__ int swz(int r);
template <> __device__ __forceinline__ int swz<128>(int r) {
  return ((r & 1) ? 4 : 0) ^ ((r & 2) ? 10 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 8 : 0);
}
template <> __device__ __forceinline__ int swz<64>(int r) {
  return ((r & 1) ? 2 : 0) ^ ((r & 2) ? 4 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 2 : 0);
}

// Element offset of chunk c of row r.
template <int D> __device__ __forceinline__ int chunk_off(int r, int c) {
  return r * D + ((c ^ swz<D>(r)) << 3);
}

// 8 elements (one 16-byte chunk) of a row.
template <int D>
__device__ __forceinline__ u32x4 read_row(const uint16_t *tile, int r, int c) {
  return *(const u32x4 *)(tile + chunk_off<D>(r, c));
}

template <int D>
__device__ __forceinline__ void write_chunk(uint16_t *tile, int r, int c, u32x4 v) {
  *(u32x4 *)(tile + chunk_off<D>(r, c)) = v;
}

// Transposed operand: lane l receives X[16c + 8*(s/4) + 4*(l/32) + s%4][n0 + l%32]
// in slot s (0..7), X being the tile (rows r0.., columns = elements of a row).
template <int D>
__device__ __forceinline__ u32x4 read_tr(const uint16_t *tile, int r0, int c, int n0, int l) {
  const int col = n0 + 16 * ((l >> 4) & 1) + 4 * (l & 3);
  const int row = r0 + 16 * c + 4 * (l >> 5) + ((l & 15) >> 2);
  const int cc = col >> 3, within = col & 7;
  const uint16_t *p0 = tile + row * D + ((cc ^ swz<D>(row)) << 3) + within;
  const uint16_t *p1 = tile + (row + 8) * D + ((cc ^ swz<D>(row + 8)) << 3) + within;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p1);
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// The same two reads from per-lane byte offsets computed once per kernel.
// With double buffering, each buffer is its own LDS variable (see BufIdx) at a
// fixed address; passing the offsets through opaque() once per step keeps the
// compiler from hoisting one full set of addresses per buffer out of the
// loop: the buffer's address then folds into the instruction's immediate
// offset, and one set of offset registers serves both buffers.
template <int D>
__device__ __forceinline__ uint32_t row_off(int r, int c) {
  return 2u * (uint32_t)chunk_off<D>(r, c);
}

// 8 elements of row (r + dr) at chunk c, with off = row_off(r, c) and dr a
// multiple of 16 (which leaves the swizzle unchanged).
template <int D>
__device__ __forceinline__ u32x4 read_row_at(const uint16_t *tile, int dr, uint32_t off) {
  return *(const u32x4 *)((const char *)(tile + dr * D) + off);
}

// Offsets of the two halves of read_tr(tile, 0, 0, n0, l); chunk c of the
// contraction is 16c rows further down (same swizzle).
template <int D>
__device__ __forceinline__ void tr_off(uint32_t o[2], int n0, int l) {
  const int col = n0 + 16 * ((l >> 4) & 1) + 4 * (l & 3);
  const int row = 4 * (l >> 5) + ((l & 15) >> 2);
  const int cc = col >> 3, within = col & 7;
  o[0] = 2u * (uint32_t)(row * D + ((cc ^ swz<D>(row)) << 3) + within);
  o[1] = 2u * (uint32_t)((row + 8) * D + ((cc ^ swz<D>(row + 8)) << 3) + within);
}

template <int D>
__device__ __forceinline__ u32x4 read_tr_at(const uint16_t *tile, int c, const uint32_t o[2]) {
  const char *base = (const char *)(tile + 16 * c * D);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + o[0]));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + o[1]));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// Max of x over the lane pair (l, l ^ 32), in every lane.  gfx950's
// v_permlane32_swap exchanges the upper 32 lanes of one register with the
// lower 32 lanes of another: with both holding x, one ends up with the lower
// half's values in all 64 lanes and the other with the upper half's, whichever
// way round; their max is the pair max.  A VALU operation, where a shuffle
// through ds_bpermute would queue behind the LDS traffic.  (The compiler's
// builtin for this instruction returns the first result twice, so it is
// written out; the nops cover the VALU write -> permlane read hazard and its
// result's first use.)
__device__ __forceinline__ float max_lane_pair(float x) {
  float a = x, b = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

// Makes the values look modified (they are not) so that nothing computed from
// them is hoisted out of the enclosing loop.
template <int N>
__device__ __forceinline__ void opaque(uint32_t (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}

// Direct global -> LDS loads of a tile of R rows of D 16-bit elements.  Each
// wave instruction fills 1 KB of LDS (lane l writes bytes [16l, 16l + 16)
// after the base the instruction names), i.e. 512/D consecutive rows, and
// lane l fetches the logical chunk that the swizzle puts at its physical
// position.  The per-lane byte offsets do not depend on the tile, so they are
// computed once (tile_offsets); a tile is then named by a uniform byte offset
// (the buffer's soffset).  Rows past the buffer's end read as zeros.  The
// loads are asynchronous: wait for vmcnt before the tile is read.
template <int D, int R, int NW>
struct TileGeom {
  static constexpr int RPI = 512 / D;   // rows per wave instruction
  static constexpr int NI = R / RPI;    // wave instructions per tile
  static constexpr int PER_WAVE = NI / NW;
  static_assert(NI % NW == 0, "tile must split evenly over the waves");
};

// Per-lane byte offsets of this wave's share of a tile (computed once).
template <int D, int R, int NW>
__device__ __forceinline__ void tile_offsets(uint32_t *voff, uint32_t rowb, int w, int l) {
  using G = TileGeom<D, R, NW>;
  const int rsub = l / (D / 8), pc = l % (D / 8);
#pragma unroll
  for (int k = 0; k < G::PER_WAVE; ++k) {
    const int row = (k * NW + w) * G::RPI + rsub;
    voff[k] = (uint32_t)row * rowb + (uint32_t)((pc ^ swz<D>(row)) << 4);
  }
}

// Issues this wave's loads of the tile whose row 0 sits at byte `tile_base`.
template <int D, int R, int NW>
__device__ __forceinline__ void tile_load(uint16_t *tile, __amdgpu_buffer_rsrc_t rs,
                                          const uint32_t *voff, uint32_t tile_base, int w) {
  using G = TileGeom<D, R, NW>;
#pragma unroll
  for (int k = 0; k < G::PER_WAVE; ++k) {
    const int r0 = (k * NW + w) * G::RPI;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void *)(tile + r0 * D), 16, voff[k],
        (int)tile_base, 0, 0);
  }
}

// Waits for this wave's outstanding global loads (including loads into LDS)
// and LDS operations, then joins the workgroup barrier.  The wait is the
// builtin, not inline asm, so that the compiler's own counter bookkeeping
// knows the loads have retired and adds no waits of its own after it; the
// barrier's memory clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void vm_wait_barrier() {
  __builtin_amdgcn_sched_barrier(0);    // no work of either side moves across
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) expcnt(7) lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Compile-time buffer index of a double-buffered tile.  Each buffer is its own
// LDS variable and every access names it statically: the compiler can then
// tell a read of the current buffer from a pending direct-to-LDS load into the
// other one, and does not make the read wait for that load.
template <int B> using BufIdx = std::integral_constant<int, B>;

// Rounds 8 accumulator registers r0..r0+7 to 16 bits: the operand slots of
// one 16-row chunk in the order read_tr uses.
template <typename T>
__device__ __forceinline__ u32x4 pack8(const f32x16 &x, int r0) {
  return u32x4{pack2<T>(x[r0 + 0], x[r0 + 1]), pack2<T>(x[r0 + 2], x[r0 + 3]),
               pack2<T>(x[r0 + 4], x[r0 + 5]), pack2<T>(x[r0 + 6], x[r0 + 7])};
}

}  // namespace fa
