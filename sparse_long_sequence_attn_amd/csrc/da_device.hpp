// Device helpers shared by the backward kernels: buffer loads with hardware
// range checks, the LDS transpose read, lane-pair reductions and the
// XCD-aware tile order.
#pragma once

#include "da_common.hpp"

namespace da {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer over [base, base + bytes): 16-byte loads at 32-bit offsets;
// offsets at or past `bytes` read as zero (gfx9 resource word 3 = 0x00020000).
__device__ inline __amdgpu_buffer_rsrc_t dev_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ inline u32x4 dev_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane m supplies 4 consecutive 16-bit elements; view them in lane order as
// a 4 x 16 matrix (rows = lanes 4j..4j+3). Lane i receives column i:
// element j = row j, column i.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;
typedef const char __attribute__((address_space(3)))* lds_cptr;
__device__ inline u32x2 dev_read_tr16(lds_cptr base, uint32_t byte_off) {
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(base + byte_off)));
}

// ---- bf16 tiles loaded straight into LDS (128-byte rows, no padding)
//
// A buffer load with the LDS bit puts lane i's 16 bytes at dst + 16 i,
// whatever offset the lane loads from (measured), and writes zeros for
// offsets at or past the buffer's range. Device pass only: the host pass
// has no such builtin and would drop the kernel's launch stub.
typedef __attribute__((address_space(3))) char* lds_ptr;
__device__ inline void dev_dma16(__amdgpu_buffer_rsrc_t r, lds_ptr dst, uint32_t off,
                                 uint32_t soff = 0) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, soff, 0, 0);
#endif
}

// Slot of 16-byte chunk c of row R: c ^ s(R), s the three bits of
// t = (R >> 1) & 7 rotated right by one. Reads of one chunk of 16
// consecutive rows fill the 16 slots of a 256-byte bank window; transpose
// reads of 4 consecutive rows (64 bytes each, rows 4m.. 4m+3) land on 4
// distinct quarters, since rows 4m and 4m + 2 differ in bit 2 of s. The
// map is its own inverse: slot j of row R holds chunk dma_slot(R, j).
__device__ inline int dma_slot(int R, int c) {
  const int t = (R >> 1) & 7;
  return c ^ (((t & 1) << 2) | (t >> 1));
}

// Stages BR rows of one tensor with NW waves: each wave issues DW loads of
// 1 KiB (8 rows); lane i of load j fetches the chunk that belongs at its
// slot. load() takes the wave index and the tile's byte offset as
// wave-uniform values (scalar registers: the offset goes in the loads'
// scalar offset field).
template <int BR, int NW>
struct DmaTile {
  static constexpr int DW = BR * 128 / 1024 / NW;
  static_assert(DW >= 1 && BR * 128 % (1024 * NW) == 0, "tile split");
  uint32_t off[DW];
  __device__ inline void init(int wv, int lane, uint32_t mbytes) {
#pragma unroll
    for (int j = 0; j < DW; ++j) {
      const int R = 8 * (DW * wv + j) + (lane >> 3);
      off[j] = (uint32_t)R * mbytes + (uint32_t)(dma_slot(R, lane & 7) * 16);
    }
  }
  __device__ inline void load(__amdgpu_buffer_rsrc_t r, lds_ptr tile, uint32_t base,
                              int wv) const {
#pragma unroll
    for (int j = 0; j < DW; ++j) dev_dma16(r, tile + (DW * wv + j) * 1024, off[j], base);
  }
};

// Byte offset, from a 16-row-aligned row of such a tile, of a lane's
// transpose read of fragment half h (rows + 8 h) of dims 32 db .. + 31: the
// lane order of tr_lane_offset (row 8 h + 4 (g >> 1) + m / 4, dims
// 32 db + 16 (g & 1) + 4 (m & 3) .. + 3 in 16-lane group g, lane m) with the
// chunk moved to its slot.
__device__ inline uint32_t dma_tr_offset(int lane, int h, int db) {
  const int m16 = lane & 15, g16 = lane >> 4;
  const int R = 8 * h + 4 * (g16 >> 1) + (m16 >> 2);
  const int dd = 16 * (g16 & 1) + 4 * (m16 & 3);
  return (uint32_t)(R * 128 + dma_slot(R, 4 * db + (dd >> 3)) * 16 + (dd & 7) * 2);
}

// The eight transpose reads of two 16-key (or 16-query) steps c = 0, 1 of
// a 32-row block: a[db][h] is the lane's address of step 0 (block base +
// dma_tr_offset), step 1 is 2048 bytes on. f[db][c] is the MFMA operand
// (h = 0 half, then h = 1). Written out with one wait at the end: the
// compiler's own transpose reads would each wait for loads still in flight
// into another buffer. Outputs are early-clobber (none may share a register
// with an address).
__device__ inline void dma_tr_read8(bf16x8 (&f)[2][2], const uint32_t (&a)[2][2]) {
  u32x2 r[8];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:2048\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %11\n\t"
      "ds_read_b64_tr_b16 %6, %10 offset:2048\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0][0]), "v"(a[0][1]), "v"(a[1][0]), "v"(a[1][1])
      : "memory");
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const u32x2 lo = r[4 * db + 2 * c], hi = r[4 * db + 2 * c + 1];
      f[db][c] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
}

__device__ inline uint32_t dev_pack_bf16(float x, float y) {
  bf16x2 p;
  p[0] = (__bf16)x;
  p[1] = (__bf16)y;
  return __builtin_bit_cast(uint32_t, p);
}

// One (pattern, batch, head, segment) unit and a tile of rows inside it.
struct UnitTile {
  int64_t b;
  int64_t seg;
  int32_t h;
  int32_t p;     // index into the sorted pattern list
  int32_t tile;  // row tile inside the segment
};

// Block id -> tile. Block ids are dealt to the XCDs round-robin (id mod
// kXcds); each XCD walks its share of every pattern's units in groups of 4
// units (their rows about fill the XCD's L2), the heaviest tiles of the
// group first; the last pattern's groups are larger (as many units as fill
// the L2), so the XCD's list ends with its shortest tiles and its workgroup
// slots drain together (decode_order). The
// heaviest tile of a unit is its last one (LAST_FIRST) or its first one,
// whichever carries the most work. Returns false for the padding blocks of
// XCDs whose list is shorter than the longest one.
template <bool LAST_FIRST, class Args>
__device__ inline bool decode_unit_tile(const Args& a, int64_t id, UnitTile* t) {
  int32_t p;
  uint32_t unit, rank;
  if (!decode_order(a, (uint32_t)id, &p, &unit, &rank)) return false;
  const uint32_t bh = fdiv(unit, a.pat[p].nseg_div);
  t->seg = unit - bh * (uint32_t)a.pat[p].nseg;
  const uint32_t b = fdiv(bh, a.h_div);
  t->h = (int32_t)(bh - b * (uint32_t)a.H);
  t->b = b;
  t->p = p;
  t->tile = LAST_FIRST ? (int32_t)((uint32_t)a.pat[p].ntile - 1u - rank) : (int32_t)rank;
  return true;
}

// Number of patterns that gather position t for head h.
template <class Args>
__device__ inline int coverage(const Args& a, uint32_t t, int32_t h) {
  int cover = 0;
  for (int i = 0; i < a.np; ++i)
    cover += compact_index(t, a.pat[i], head_offset(h, a.pat[i].r)) >= 0;
  return cover;
}

}  // namespace da
