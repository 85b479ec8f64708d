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
// group first; the last pattern's units form one group, so the XCD's list
// ends with its shortest tiles and its workgroup slots drain together. The
// heaviest tile of a unit is its last one (LAST_FIRST) or its first one,
// whichever carries the most work. Returns false for the padding blocks of
// XCDs whose list is shorter than the longest one.
template <bool LAST_FIRST, class Args>
__device__ inline bool decode_unit_tile(const Args& a, int64_t id, UnitTile* t) {
  const int32_t x = (int32_t)(id % kXcds);
  int64_t slot = id / kXcds;
  for (int p = 0; p < a.np; ++p) {
    const int64_t u0 = a.unit_start[p], u1 = a.unit_start[p + 1];
    const int64_t first = u0 + (((x - u0) % kXcds) + kXcds) % kXcds;
    const int64_t cnt = first < u1 ? (u1 - first + kXcds - 1) / kXcds : 0;
    const int64_t nt = a.pat[p].ntile;
    if (slot < cnt * nt) {
      const int64_t G = p == a.np - 1 ? (cnt > 0 ? cnt : 1) : 4;
      const int64_t gfull = cnt / G;
      int64_t gi = slot / (G * nt), gsz = G;
      if (gi >= gfull) {
        gi = gfull;
        gsz = cnt - gfull * G;
      }
      const int64_t r0 = slot - gi * G * nt;
      const int32_t k = (int32_t)(r0 / gsz);
      const int64_t lu = gi * G + r0 % gsz;
      const int64_t rem = first + lu * kXcds - u0;
      const int64_t nseg = a.pat[p].nseg;
      t->seg = rem % nseg;
      const int64_t bh = rem / nseg;
      t->h = (int32_t)(bh % a.H);
      t->b = bh / a.H;
      t->p = p;
      t->tile = LAST_FIRST ? (int32_t)(nt - 1 - k) : k;
      return true;
    }
    slot -= cnt * nt;
  }
  return false;
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
