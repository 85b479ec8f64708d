// Backward pass of dilated attention for gfx950 (MI355X).
//
// LongNet is trained (LongNet package README, "Key Advantages": training
// runs and the distributed trainer; LONGNET blog, "Token expansion reaches
// 1 billion+": training split along the sequence), so the path needs the
// gradients of the forward pass. The merged output of a row is one softmax
// over the multiset of (pattern, key) pairs that its covering patterns give
// it (the log-sum-exp merge reading), so with the merged lse and
// D = dout . out of each row, every pattern's segments contribute
// independently:
//   P = exp(scale q.k - lse),  dP = dout . v,  dS = P (dP - D),
//   dq += scale dS k,  dk += scale dS^T q,  dv += P^T dout,
// summed over the patterns that gather a row.
//
// Kernels:
//  * bwd_short_kernel: when every segment gathers at most 32 rows, one wave
//    per (pattern, batch, head, segment) unit computes D, dq, dk and dv at
//    once; the three kernels below then have nothing to do.
//  * bwd_prep_kernel: D for every row.
//  * bwd_kv_kernel: one workgroup per tile of 128 gathered keys (4 waves of
//    32) of one unit. Each wave keeps the dK^T, dV^T accumulators of its 32
//    keys in registers, reads its keys' K and V fragments from LDS (bf16;
//    registers for fp32) and streams the unit's query rows (Q, dout, lse, D)
//    through LDS, double buffered, 32 rows per stage.
//    S = Q K^T puts one key in each lane and 16 of its queries in registers,
//    which is the B-operand layout of dV^T += dout^T P and dK^T += Q^T dS;
//    their A operands (8 queries of one dimension per lane) come from the
//    LDS transpose read.
//  * bwd_q_kernel: one workgroup per tile of 128 gathered queries, in the
//    forward kernel's layout (S^T = K Q^T: one query per lane), K and V
//    streamed through LDS; dQ^T += K^T dS^T takes K^T from the transpose read.
//  * bwd_merge_kernel: rows several patterns gather add up their partials
//    (stored in the gradients' dtype, summed in fp32); rows no pattern
//    gathers get zero gradients.
// bf16 inputs use v_mfma_f32_32x32x16_bf16 with P and dS rounded to bf16 as
// MFMA operands; fp32 inputs use v_mfma_f32_32x32x2_f32 throughout.
//
// Rows past a segment's last gathered row load as zeros (buffer range
// checks) and get lse = +inf and D = 0, so their P and dS are exactly 0; keys
// past it have K = V = 0 and add nothing to dQ, and their own dK, dV are
// never stored.
#include <type_traits>

#include "da_bwd.hpp"
#include "da_device.hpp"
#include "kernels.hpp"

namespace da {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

// LDS row stride in elements: bf16 rows of 72 elements (144 bytes), so the
// 16 lanes the LDS serves together when reading 16-byte chunks of 16
// consecutive rows hit distinct bank groups, and the transpose read applies;
// fp32 rows of 65 floats.
template <bool BF>
constexpr int lds_stride() {
  return BF ? kDh + 8 : kDh + 1;
}

// Byte offset of a lane's LDS transpose read inside a 16 x 32 block of a
// bf16 tile with row stride ST: in 16-lane group g (n = 16 (g & 1) + i,
// hh = g >> 1) lane m points at row 8 h' + 4 hh + m / 4 (h' = 0 for the first
// read, 1 for the second, 8 rows further), columns 16 (g & 1) + 4 (m & 3) ..
// +3; the read then hands lane i the four rows of column i. Two reads give a
// lane rows {0..3, 8..11} + 4 hh of its column: the k order
// 16c + 8(e / 4) + 4hh + e % 4 that matches the MFMA output layout.
template <int ST>
__device__ inline uint32_t tr_lane_offset(int lane) {
  const int m16 = lane & 15, g16 = lane >> 4;
  return (uint32_t)((4 * (g16 >> 1) + (m16 >> 2)) * ST + 16 * (g16 & 1) + 4 * (m16 & 3)) * 2;
}

__device__ inline bf16x8 tr_fragment(lds_cptr base, uint32_t off, int ST) {
  const u32x2 lo = dev_read_tr16(base, off);
  const u32x2 hi = dev_read_tr16(base, off + 8 * ST * 2);
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

__device__ inline bf16x8 to_bf16x8(const float* x) {
  u32x4 u;
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = dev_pack_bf16(x[2 * i], x[2 * i + 1]);
  return __builtin_bit_cast(bf16x8, u);
}

// Gathered-row geometry of one tile's unit.
struct UnitGeom {
  int32_t r, off, L;
  int64_t wp, seg0, headbase, rs, bh;
  uint32_t mbytes, range;
};

template <class T>
__device__ inline UnitGeom unit_geom(const BwdArgs& a, const UnitTile& tl) {
  UnitGeom g;
  const PatDev& P = a.pat[tl.p];
  g.r = P.r;
  g.wp = P.wp;
  g.off = head_offset(tl.h, g.r);
  g.L = rows_gathered(g.wp, g.off, g.r);
  g.rs = (int64_t)a.H * kDh;
  g.seg0 = tl.seg * g.wp;
  g.headbase = tl.b * a.N * g.rs + (int64_t)tl.h * kDh;
  g.bh = tl.b * a.H + tl.h;
  // gathered row m of the unit starts m * mbytes bytes after row 0; the host
  // keeps these offsets (plus one tile of overrun) below 2^31
  g.mbytes = (uint32_t)((int64_t)g.r * g.rs * (int64_t)sizeof(T));
  g.range = (uint32_t)(g.L - 1) * g.mbytes + (uint32_t)(kDh * sizeof(T));
  return g;
}

// Register fragments of gathered row m of one tensor as an MFMA operand
// with the row in the lane: bf16 - dims 16 ks + 8 hh .. +7 for ks = 0..3;
// fp32 - dim 2 ks + hh for ks = 0..31.
template <bool BF>
struct RowFrag {
  typename std::conditional<BF, bf16x8, float>::type x[BF ? 4 : 32];
  __device__ inline void load(__amdgpu_buffer_rsrc_t rsrc, uint32_t row_off, int hh) {
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        x[ks] = __builtin_bit_cast(bf16x8, dev_load16(rsrc, row_off + (16 * ks + 8 * hh) * 2));
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const f32x4 v = __builtin_bit_cast(f32x4, dev_load16(rsrc, row_off + 16 * c));
        x[2 * c] = hh ? v[1] : v[0];
        x[2 * c + 1] = hh ? v[3] : v[2];
      }
    }
  }
  // the same fragments from a row staged in LDS (row stride lds_stride<BF>)
  template <class T>
  __device__ inline void load_lds(const T* row, int hh) {
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        x[ks] = *reinterpret_cast<const bf16x8*>(row + 16 * ks + 8 * hh);
    } else {
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) x[ks] = row[2 * ks + hh];
    }
  }
};

// Stages R gathered rows of two tensors (16-byte chunks: global ->
// registers -> LDS) for a workgroup of NT threads.
template <bool BF, int R, int NT>
struct PairStager {
  using T = typename std::conditional<BF, __bf16, float>::type;
  static constexpr int ST = lds_stride<BF>();
  static constexpr int kChunksPerRow = kDh * (int)sizeof(T) / 16;
  static constexpr int CK = R * kChunksPerRow / NT;
  static_assert(CK >= 1 && R * kChunksPerRow % NT == 0, "tile too small for the workgroup");
  u32x4 ra[CK], rb[CK];
  uint32_t off[CK];

  __device__ inline void init(int tid, uint32_t mbytes) {
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * NT;
      off[i] = (uint32_t)(c / kChunksPerRow) * mbytes + (uint32_t)(c % kChunksPerRow) * 16;
    }
  }
  __device__ inline void load(__amdgpu_buffer_rsrc_t sa, __amdgpu_buffer_rsrc_t sb, uint32_t base) {
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      ra[i] = dev_load16(sa, base + off[i]);
      rb[i] = dev_load16(sb, base + off[i]);
    }
  }
  __device__ inline void store_first(int tid, T* A) const {
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * NT;
      const int row = c / kChunksPerRow, ch = c % kChunksPerRow;
      if constexpr (BF) {
        *reinterpret_cast<u32x4*>(A + row * ST + ch * 8) = ra[i];
      } else {
        float* da = reinterpret_cast<float*>(A) + row * ST + 4 * ch;
#pragma unroll
        for (int e = 0; e < 4; ++e) da[e] = __uint_as_float(ra[i][e]);
      }
    }
  }
  __device__ inline void store(int tid, T* A, T* B) const {
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * NT;
      const int row = c / kChunksPerRow, ch = c % kChunksPerRow;
      if constexpr (BF) {
        *reinterpret_cast<u32x4*>(A + row * ST + ch * 8) = ra[i];
        *reinterpret_cast<u32x4*>(B + row * ST + ch * 8) = rb[i];
      } else {
        float* da = reinterpret_cast<float*>(A) + row * ST + 4 * ch;
        float* db = reinterpret_cast<float*>(B) + row * ST + 4 * ch;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          da[e] = __uint_as_float(ra[i][e]);
          db[e] = __uint_as_float(rb[i][e]);
        }
      }
    }
  }
};

// Writes one lane's half of a gradient row held in MFMA output layout (two
// 32-dim blocks; register 4g + e of block db is dim db*32 + 8g + 4hh + e),
// multiplied by mul, either into the final tensor or into a partial row
// (the partials have the gradients' dtype: 64 contiguous elements per row).
template <bool BF>
__device__ inline void put_row(void* dst_tensor, int64_t elem_off, const f32x16 (&acc)[2],
                               float mul, int hh) {
  using T = typename std::conditional<BF, __bf16, float>::type;
  T* dst = reinterpret_cast<T*>(dst_tensor) + elem_off + 4 * hh;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + 8 * g;
      if constexpr (BF) {
        *reinterpret_cast<u32x2*>(dst + d) =
            u32x2{dev_pack_bf16(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul),
                  dev_pack_bf16(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
      } else {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * g + e] * mul;
        *reinterpret_cast<f32x4*>(dst + d) = x;
      }
    }
}

// Row-contiguous writes for the short-segment kernel (one wave per unit of
// at most 32 rows, bound by its memory traffic): each lane stages its
// half row (MFMA layout) in LDS, then 16 lanes write each of the wave's 32
// rows as one contiguous line - 128 bytes of bf16 (256 of fp32) - instead of
// 8-byte pieces of 32 rows per store.
constexpr int kStageStride = kDh + 4;  // floats; conflict-free 16-byte writes
constexpr int kStageBytes = 32 * kStageStride * 4 + 32 * 8;

__device__ inline void stage_row(float* srow, const f32x16 (&acc)[2], float mul, int n, int hh) {
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * g + e] * mul;
      *reinterpret_cast<f32x4*>(srow + n * kStageStride + db * 32 + 8 * g + 4 * hh) = x;
    }
}

// Rows of kind 1 go to final + pos * rs, rows of kind 2 to partial + R * kDh
// (the wave's first gathered row at partial, in the gradients' dtype); kind 0
// rows are skipped.
template <bool BF>
__device__ inline void write_rows(
    const float* srow, const int32_t* mpos, const int32_t* mkind, void* final_base, int64_t rs,
    typename std::conditional<BF, __bf16, float>::type* partial, int lane) {
  using T = typename std::conditional<BF, __bf16, float>::type;
  const int sr = lane >> 4, sc = lane & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int R = 4 * i + sr;
    const int32_t kind = mkind[R];
    if (kind == 0) continue;
    const f32x4 x = *reinterpret_cast<const f32x4*>(srow + R * kStageStride + 4 * sc);
    T* dst = kind == 1 ? reinterpret_cast<T*>(final_base) + (int64_t)mpos[R] * rs + 4 * sc
                       : partial + (int64_t)R * kDh + 4 * sc;
    if constexpr (BF)
      *reinterpret_cast<u32x2*>(dst) = u32x2{dev_pack_bf16(x[0], x[1]), dev_pack_bf16(x[2], x[3])};
    else
      *reinterpret_cast<f32x4*>(dst) = x;
  }
}

// ---------------------------------------------------------------- dK, dV

template <int NW, bool CAUSAL, bool BF>
// bf16: at least 3 waves per SIMD (the fragments of K and V live in LDS)
__global__ __launch_bounds__(NW * 64, BF ? 3 : 1) void bwd_kv_kernel(const BwdArgs a) {
  static_assert(NW == 4, "segments of at most 32 rows take bwd_short_kernel");
  using T = typename std::conditional<BF, __bf16, float>::type;
  constexpr int BQ = 32;  // query rows per LDS tile
  constexpr int QBT = BQ / 32;
  constexpr int NT = 64 * NW;
  constexpr int ST = lds_stride<BF>();
  // bf16: Q and dout tiles loaded straight into LDS (128-byte rows, chunks
  // at dma_slot); fp32: staged through registers into padded rows
  constexpr int kTileElems = BF ? BQ * kDh : BQ * ST;
  constexpr int kTileBytes = kTileElems * (int)sizeof(T);
  constexpr int kBufBytes = 2 * kTileBytes + 2 * BQ * 4;  // Q, dout, lse2, D
  static_assert(kTileBytes % 16 == 0, "LDS alignment");
  // bf16: the workgroup's 32 * NW V rows stay in LDS (128-byte rows, 16-byte
  // chunk j of row x at slot j ^ ((x >> 1) & 7)) instead of registers
  constexpr int kVBytes = BF ? 32 * NW * kDh * 2 : 0;
  __shared__ __attribute__((aligned(16))) char smem[2 * kBufBytes + 2 * kVBytes];
  T* const Vl = reinterpret_cast<T*>(smem + 2 * kBufBytes);
  T* const Kl = reinterpret_cast<T*>(smem + 2 * kBufBytes + kVBytes);

  UnitTile tl;
  if (!decode_unit_tile<false>(a, blockIdx.x, &tl)) return;
  const UnitGeom g = unit_geom<T>(a, tl);
  const int32_t k0 = tl.tile * 32 * NW;
  if (k0 >= g.L) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int64_t rowbase = g.headbase + (g.seg0 + g.off) * g.rs;
  const auto rq = dev_rsrc(reinterpret_cast<const T*>(a.q) + rowbase, g.range);
  const auto rk = dev_rsrc(reinterpret_cast<const T*>(a.k) + rowbase, g.range);
  const auto rv = dev_rsrc(reinterpret_cast<const T*>(a.v) + rowbase, g.range);
  const auto rdo = dev_rsrc(reinterpret_cast<const T*>(a.dout) + rowbase, g.range);
  const float* lse_row = a.lse + g.bh * a.N;
  const float* d_row = a.dvec + g.bh * a.N;

  // this wave's index and first key, wave-uniform (scalar branches below)
  const int wvs = __builtin_amdgcn_readfirstlane(wv);
  const int32_t kw0 = __builtin_amdgcn_readfirstlane(k0 + 32 * wv);
  const int32_t mk = kw0 + n;  // this lane's key
  RowFrag<BF> kf, vf;                // B operands of S = Q K^T and dP = dout V^T
  kf.load(rk, (uint32_t)mk * g.mbytes, hh);
  vf.load(rv, (uint32_t)mk * g.mbytes, hh);
  const int vrow = wv * 32 + n;
  if constexpr (BF) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int o = vrow * kDh + (((2 * ks + hh) ^ ((vrow >> 1) & 7)) << 3);
      *reinterpret_cast<bf16x8*>(Vl + o) = vf.x[ks];
      *reinterpret_cast<bf16x8*>(Kl + o) = kf.x[ks];
    }
  }

  f32x16 dK[2], dV[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) dK[db][v] = dV[db][v] = 0.f;

  // query tiles: from this workgroup's first key (causal) or row 0
  const int32_t qstart = CAUSAL ? k0 : 0;  // a multiple of BQ
  const int32_t nqt = (g.L - qstart + BQ - 1) / BQ;

  PairStager<BF, BF ? NT / 8 : BQ, NT> stg;  // fp32 only
  DmaTile<BQ, NW> dmt;                      // bf16 only
  if constexpr (BF)
    dmt.init(wv, lane, g.mbytes);
  else
    stg.init(tid, g.mbytes);
  // lse and D of query row tid of the next tile; lse is scaled to log2 only
  // when stored, since using a loaded value right away would make the wave
  // wait for the tile loads issued just before it. bf16: the Q and dout
  // tiles go into buffer buf directly.
  float lreg = 0.f, dreg = 0.f;
  auto load_tile = [&](int t, int buf) {
    const int32_t m0 = qstart + t * BQ;
    if constexpr (BF) {
      const lds_ptr qt = (lds_ptr)smem + buf * kBufBytes;
      dmt.load(rq, qt, (uint32_t)m0 * g.mbytes, wvs);
      dmt.load(rdo, qt + kTileBytes, (uint32_t)m0 * g.mbytes, wvs);
    } else {
      stg.load(rq, rdo, (uint32_t)m0 * g.mbytes);
    }
    if (tid < BQ) {
      const int32_t m = m0 + tid;
      lreg = INFINITY;
      dreg = 0.f;
      if (m < g.L) {
        const int64_t pos = g.seg0 + g.off + (int64_t)m * g.r;
        lreg = lse_row[pos];
        dreg = d_row[pos];
      }
    }
  };
  auto store_tile = [&](int buf) {
    char* base = smem + buf * kBufBytes;
    if constexpr (!BF)
      stg.store(tid, reinterpret_cast<T*>(base), reinterpret_cast<T*>(base + kTileBytes));
    if (tid < BQ) {
      float* ls = reinterpret_cast<float*>(base + 2 * kTileBytes);
      ls[tid] = lreg * kLog2e;
      ls[BQ + tid] = -dreg;  // -D: the dP products accumulate onto it
    }
  };

  const float sl2 = a.sl2;
  uint32_t trq[2][2];  // bf16: transpose-read offsets (dma_tr_offset)
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h) trq[db][h] = BF ? dma_tr_offset(lane, h, db) : 0u;

  auto compute = [&](int buf, int t) {
    const char* base = smem + buf * kBufBytes;
    const T* Qs = reinterpret_cast<const T*>(base);
    const T* Ds = reinterpret_cast<const T*>(base + kTileBytes);
    const float* ls = reinterpret_cast<const float*>(base + 2 * kTileBytes);
    const float* ndd = ls + BQ;  // -D per query row
#pragma unroll
    for (int qb = 0; qb < QBT; ++qb) {
      const int32_t qs = qstart + t * BQ + 32 * qb;  // first query of the block
      if (qs >= g.L) break;
      if (CAUSAL && qs < kw0) continue;  // 32-aligned: every query precedes every key
      const int row = qb * 32 + n;
      // dP starts at -D of its query (register v: query qb*32 + 8(v/4) +
      // 4hh + v%4), so the products leave dP - D for dS = P (dP - D)
      f32x16 S, dP;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 nd4 = *reinterpret_cast<const f32x4*>(ndd + qb * 32 + 8 * gq + 4 * hh);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          S[4 * gq + j] = 0.f;
          dP[4 * gq + j] = nd4[j];
        }
      }
      if constexpr (BF) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int oq = row * kDh + dma_slot(row, 2 * ks + hh) * 8;
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qs + oq);
          const bf16x8 da = *reinterpret_cast<const bf16x8*>(Ds + oq);
          const int o = vrow * kDh + (((2 * ks + hh) ^ ((vrow >> 1) & 7)) << 3);
          const bf16x8 kb = *reinterpret_cast<const bf16x8*>(Kl + o);
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb, S, 0, 0, 0);
          const bf16x8 vb = *reinterpret_cast<const bf16x8*>(Vl + o);
          dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vb, dP, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
          const float qa = reinterpret_cast<const float*>(Qs)[row * ST + 2 * ks + hh];
          const float da = reinterpret_cast<const float*>(Ds)[row * ST + 2 * ks + hh];
          S = __builtin_amdgcn_mfma_f32_32x32x2f32(qa, kf.x[ks], S, 0, 0, 0);
          dP = __builtin_amdgcn_mfma_f32_32x32x2f32(da, vf.x[ks], dP, 0, 0, 0);
        }
      }
      // register v: query qb*32 + 8(v/4) + 4hh + v%4 of the tile, key n
      float pv[16], sv[16];
      u32x4 pk[2], sk[2];  // bf16 P and dS, packed as they are formed
      auto probs = [&](bool diag) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int qi = qb * 32 + 8 * gq + 4 * hh;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + qi);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int v = 4 * gq + j;
            float p = __builtin_amdgcn_exp2f(fmaf(S[v], sl2, -l4[j]));
            if (diag && 8 * gq + 4 * hh + j < n) p = 0.f;
            pv[v] = p;
            sv[v] = p * dP[v];
          }
          if constexpr (BF) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int v = 4 * gq + 2 * j;
              pk[gq >> 1][2 * (gq & 1) + j] = dev_pack_bf16(pv[v], pv[v + 1]);
              sk[gq >> 1][2 * (gq & 1) + j] = dev_pack_bf16(sv[v], sv[v + 1]);
            }
          }
        }
      };
      if (CAUSAL && qs == kw0)  // the diagonal block: keys after their query masked
        probs(true);
      else
        probs(false);
      if constexpr (BF) {
        const uint32_t qaddr = (uint32_t)reinterpret_cast<uintptr_t>((lds_ptr)smem) +
                               (uint32_t)(buf * kBufBytes + qb * 32 * 128);
        uint32_t ad[2][2], aq[2][2];
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            aq[db][h] = qaddr + trq[db][h];
            ad[db][h] = aq[db][h] + kTileBytes;
          }
        bf16x8 dfr[2][2], qfr[2][2];  // dout^T, Q^T fragments [db][c]
        dma_tr_read8(dfr, ad);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pk[c]);
#pragma unroll
          for (int db = 0; db < 2; ++db)
            dV[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dfr[db][c], pb, dV[db], 0, 0, 0);
        }
        dma_tr_read8(qfr, aq);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 sb = __builtin_bit_cast(bf16x8, sk[c]);
#pragma unroll
          for (int db = 0; db < 2; ++db)
            dK[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qfr[db][c], sb, dK[db], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int qi = qb * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
            const float dov = reinterpret_cast<const float*>(Ds)[qi * ST + db * 32 + n];
            const float qv = reinterpret_cast<const float*>(Qs)[qi * ST + db * 32 + n];
            dV[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(dov, pv[v], dV[db], 0, 0, 0);
            dK[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(qv, sv[v], dK[db], 0, 0, 0);
          }
      }
    }
  };

  load_tile(0, 0);
  store_tile(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // bf16: unrolled by two so each step's buffer is a compile-time constant
  auto step = [&](auto bufc, int t) {
    const int buf = bufc;
    // the other buffer was last read before the previous barrier
    if (t + 1 < nqt) load_tile(t + 1, buf ^ 1);
    compute(buf, t);
    if (t + 1 < nqt) store_tile(buf ^ 1);
    if constexpr (BF) __builtin_amdgcn_s_waitcnt(0);  // this wave's tile loads have landed
    __syncthreads();
  };
  if constexpr (BF) {
    for (int t = 0; t < nqt; t += 2) {
      step(std::integral_constant<int, 0>{}, t);
      if (t + 1 < nqt) step(std::integral_constant<int, 1>{}, t + 1);
    }
  } else {  // the fp32 tiles keep the rolled loop: unrolled, they spill
    for (int t = 0; t < nqt; ++t) step(t & 1, t);
  }

  const PatDev& P = a.pat[tl.p];
  const int64_t slots = P.units * P.lmax;
  const int64_t prow0 = (g.bh * P.nseg + tl.seg) * P.lmax;  // the unit's first slot
  if (mk >= g.L) return;
  const int64_t pos = g.seg0 + g.off + (int64_t)mk * g.r;
  if (coverage(a, (uint32_t)pos, tl.h) == 1) {
    const int64_t e = g.headbase + pos * g.rs;
    put_row<BF>(a.dk, e, dK, a.scale, hh);
    put_row<BF>(a.dv, e, dV, 1.f, hh);
  } else {
    put_row<BF>(a.ws + P.po_off, (slots + prow0 + mk) * kDh, dK, a.scale, hh);
    put_row<BF>(a.ws + P.po_off, (2 * slots + prow0 + mk) * kDh, dV, 1.f, hh);
  }
}

// ---------------------------------------------------------------- dQ

template <int NW, bool CAUSAL, bool BF>
__global__ __launch_bounds__(NW * 64, BF ? 4 : 1) void bwd_q_kernel(const BwdArgs a) {
  static_assert(NW == 4, "segments of at most 32 rows take bwd_short_kernel");
  using T = typename std::conditional<BF, __bf16, float>::type;
  constexpr int BK = 64;  // key rows per LDS tile
  constexpr int KBT = BK / 32;
  constexpr int NT = 64 * NW;
  constexpr int ST = lds_stride<BF>();
  // bf16: K and V tiles loaded straight into LDS (128-byte rows, chunks at
  // dma_slot); fp32: staged through registers into padded rows
  constexpr int kTileBytes = BF ? BK * kDh * 2 : BK * ST * (int)sizeof(T);
  constexpr int kBufBytes = 2 * kTileBytes;  // K, V
  static_assert(kTileBytes % 16 == 0, "LDS alignment");
  __shared__ __attribute__((aligned(16))) char smem[2 * kBufBytes];

  UnitTile tl;
  if (!decode_unit_tile<CAUSAL>(a, blockIdx.x, &tl)) return;
  const UnitGeom g = unit_geom<T>(a, tl);
  const int32_t q0 = tl.tile * 32 * NW;
  if (q0 >= g.L) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int64_t rowbase = g.headbase + (g.seg0 + g.off) * g.rs;
  const auto rq = dev_rsrc(reinterpret_cast<const T*>(a.q) + rowbase, g.range);
  const auto rk = dev_rsrc(reinterpret_cast<const T*>(a.k) + rowbase, g.range);
  const auto rv = dev_rsrc(reinterpret_cast<const T*>(a.v) + rowbase, g.range);
  const auto rdo = dev_rsrc(reinterpret_cast<const T*>(a.dout) + rowbase, g.range);

  // this wave's index and first query, wave-uniform (scalar branches below)
  const int wvs = __builtin_amdgcn_readfirstlane(wv);
  const int32_t qw0 = __builtin_amdgcn_readfirstlane(q0 + 32 * wv);
  const int32_t mq = qw0 + n;  // this lane's query
  RowFrag<BF> qf, df;                // B operands of S^T = K Q^T and dP^T = V dout^T
  qf.load(rq, (uint32_t)mq * g.mbytes, hh);
  df.load(rdo, (uint32_t)mq * g.mbytes, hh);
  float l2 = INFINITY, dd = 0.f;
  int64_t pos = 0;
  if (mq < g.L) {
    pos = g.seg0 + g.off + (int64_t)mq * g.r;
    l2 = a.lse[g.bh * a.N + pos] * kLog2e;
    dd = a.dvec[g.bh * a.N + pos];
  }

  f32x16 dQ[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) dQ[db][v] = 0.f;

  const int32_t qend_wg = min(g.L, q0 + 32 * NW);
  const int32_t nkt = CAUSAL ? (qend_wg + BK - 1) / BK : (g.L + BK - 1) / BK;
  const int32_t qend_w = min(g.L, qw0 + 32);
  const int32_t nkt_w =
      __builtin_amdgcn_readfirstlane(qw0 >= g.L ? 0 : (CAUSAL ? (qend_w + BK - 1) / BK : nkt));

  PairStager<BF, BF ? NT / 8 : BK, NT> stg;  // fp32 only
  DmaTile<BK, NW> dmt;                      // bf16 only
  if constexpr (BF)
    dmt.init(wv, lane, g.mbytes);
  else
    stg.init(tid, g.mbytes);
  // bf16: tile t into buffer buf; fp32: tile t into registers
  auto load_tile = [&](int t, int buf) {
    if constexpr (BF) {
      const lds_ptr kt = (lds_ptr)smem + buf * kBufBytes;
      dmt.load(rk, kt, (uint32_t)(t * BK) * g.mbytes, wvs);
      dmt.load(rv, kt + kTileBytes, (uint32_t)(t * BK) * g.mbytes, wvs);
    } else {
      stg.load(rk, rv, (uint32_t)(t * BK) * g.mbytes);
    }
  };
  auto store_tile = [&](int buf) {
    if constexpr (!BF) {
      char* base = smem + buf * kBufBytes;
      stg.store(tid, reinterpret_cast<T*>(base), reinterpret_cast<T*>(base + kTileBytes));
    }
  };

  const float sl2 = a.sl2;
  uint32_t trk[2][2];  // bf16: transpose-read offsets (dma_tr_offset)
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h) trk[db][h] = BF ? dma_tr_offset(lane, h, db) : 0u;

  auto compute = [&](int buf, int t) {
    const char* base = smem + buf * kBufBytes;
    const T* Ks = reinterpret_cast<const T*>(base);
    const T* Vs = reinterpret_cast<const T*>(base + kTileBytes);
#pragma unroll
    for (int kb = 0; kb < KBT; ++kb) {
      const int32_t kb0 = t * BK + 32 * kb;  // first key of the block
      if (kb0 >= g.L) break;
      if (CAUSAL && kb0 > qw0) break;  // 32-aligned: every key follows every query
      const int row = kb * 32 + n;
      f32x16 S, dP;
#pragma unroll
      for (int v = 0; v < 16; ++v) S[v] = dP[v] = 0.f;
      if constexpr (BF) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int o = row * kDh + dma_slot(row, 2 * ks + hh) * 8;
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + o);
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vs + o);
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf.x[ks], S, 0, 0, 0);
          dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df.x[ks], dP, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
          const float ka = reinterpret_cast<const float*>(Ks)[row * ST + 2 * ks + hh];
          const float va = reinterpret_cast<const float*>(Vs)[row * ST + 2 * ks + hh];
          S = __builtin_amdgcn_mfma_f32_32x32x2f32(ka, qf.x[ks], S, 0, 0, 0);
          dP = __builtin_amdgcn_mfma_f32_32x32x2f32(va, df.x[ks], dP, 0, 0, 0);
        }
      }
      // register v: key kb0 + 8(v/4) + 4hh + v%4, query mq
      float sv[16];
      auto probs = [&](bool diag) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float p = __builtin_amdgcn_exp2f(fmaf(S[v], sl2, -l2));
          if (diag && 8 * (v >> 2) + 4 * hh + (v & 3) > n) p = 0.f;
          sv[v] = p * (dP[v] - dd);
        }
      };
      if (CAUSAL && kb0 == qw0)  // the diagonal block: keys after the query masked
        probs(true);
      else
        probs(false);
      if constexpr (BF) {
        const uint32_t kaddr = (uint32_t)reinterpret_cast<uintptr_t>((lds_ptr)smem) +
                               (uint32_t)(buf * kBufBytes + kb * 32 * 128);
        uint32_t ad[2][2];
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int h = 0; h < 2; ++h) ad[db][h] = kaddr + trk[db][h];
        bf16x8 kfr[2][2];
        dma_tr_read8(kfr, ad);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 sb = to_bf16x8(sv + 8 * c);
#pragma unroll
          for (int db = 0; db < 2; ++db)
            dQ[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[db][c], sb, dQ[db], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int ki = kb * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
            const float kv = reinterpret_cast<const float*>(Ks)[ki * ST + db * 32 + n];
            dQ[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv, sv[v], dQ[db], 0, 0, 0);
          }
      }
    }
  };

  load_tile(0, 0);
  store_tile(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // bf16: unrolled by two so each step's buffer is a compile-time constant
  // (LDS reads then carry the buffer offset as an immediate)
  auto step = [&](auto bufc, int t) {
    const int buf = bufc;
    // the other buffer was last read before the previous barrier
    if (t + 1 < nkt) load_tile(t + 1, buf ^ 1);
    if (t < nkt_w) compute(buf, t);
    if (t + 1 < nkt) store_tile(buf ^ 1);
    if constexpr (BF) __builtin_amdgcn_s_waitcnt(0);  // this wave's tile loads have landed
    __syncthreads();
  };
  if constexpr (BF) {
    for (int t = 0; t < nkt; t += 2) {
      step(std::integral_constant<int, 0>{}, t);
      if (t + 1 < nkt) step(std::integral_constant<int, 1>{}, t + 1);
    }
  } else {  // the fp32 tiles keep the rolled loop: unrolled, they spill
    for (int t = 0; t < nkt; ++t) step(t & 1, t);
  }

  const PatDev& P = a.pat[tl.p];
  const int64_t prow0 = (g.bh * P.nseg + tl.seg) * P.lmax;  // the unit's first slot
  if (mq >= g.L) return;
  if (coverage(a, (uint32_t)pos, tl.h) == 1) {
    put_row<BF>(a.dq, g.headbase + pos * g.rs, dQ, a.scale, hh);
  } else {
    put_row<BF>(a.ws + P.po_off, (prow0 + mq) * kDh, dQ, a.scale, hh);
  }
}

// ---------------------------------------------------------------- qk_norm helpers

// Layer norm of the staged rows of one tensor in registers (chunk i of this
// lane: row (lane + 64 i) / CPR, chunk lane % CPR; a row's chunks sit in CPR
// consecutive lanes): (x - mean) / sqrt(var + eps) * gain + bias, statistics
// in fp32 over the row's 64 values. The lane holding chunk 0 of a row
// records its mean and rstd. Rows from L on (past the segment's gathered
// rows) stay zero, as the unnormalised path leaves them.
template <bool BF, int CK>
__device__ inline void qkn_normalize(u32x4 (&r)[CK], const void* gain, const void* bias,
                                     float eps, int L, int lane, float* mean_out,
                                     float* rstd_out) {
  constexpr int CPR = BF ? 8 : 16;  // chunks per row
  constexpr int VPC = BF ? 8 : 4;   // values per chunk
  const int d0 = (lane % CPR) * VPC;
  float gv[VPC], bv[VPC];
#pragma unroll
  for (int e = 0; e < VPC; ++e) {
    if constexpr (BF) {
      gv[e] = (float)reinterpret_cast<const __bf16*>(gain)[d0 + e];
      bv[e] = (float)reinterpret_cast<const __bf16*>(bias)[d0 + e];
    } else {
      gv[e] = reinterpret_cast<const float*>(gain)[d0 + e];
      bv[e] = reinterpret_cast<const float*>(bias)[d0 + e];
    }
  }
#pragma unroll
  for (int i = 0; i < CK; ++i) {
    float x[VPC];
#pragma unroll
    for (int e = 0; e < VPC; ++e) {
      if constexpr (BF)
        x[e] = __uint_as_float((e & 1) ? (r[i][e / 2] & 0xffff0000u) : (r[i][e / 2] << 16));
      else
        x[e] = __uint_as_float(r[i][e]);
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < VPC; ++e) s += x[e];
#pragma unroll
    for (int m = 1; m < CPR; m *= 2) s += __shfl_xor(s, m);
    const float mu = s * (1.f / kDh);
    float v = 0.f;
#pragma unroll
    for (int e = 0; e < VPC; ++e) v = fmaf(x[e] - mu, x[e] - mu, v);
#pragma unroll
    for (int m = 1; m < CPR; m *= 2) v += __shfl_xor(v, m);
    const float rstd = __builtin_amdgcn_rsqf(v * (1.f / kDh) + eps);
    const int row = (lane + 64 * i) / CPR;
    if (lane % CPR == 0) {
      mean_out[row] = mu;
      rstd_out[row] = rstd;
    }
    const float keep = row < L ? 1.f : 0.f;
#pragma unroll
    for (int e = 0; e < VPC; ++e) x[e] = fmaf((x[e] - mu) * rstd, gv[e], bv[e]) * keep;
#pragma unroll
    for (int e = 0; e < VPC; ++e) {
      if constexpr (BF) {
        if (e & 1) r[i][e / 2] = dev_pack_bf16(x[e - 1], x[e]);
      } else {
        r[i][e] = __float_as_uint(x[e]);
      }
    }
  }
}

// The un-normalised input values write_rows_qkn needs, in its layout: row
// 4 i + lane / 16, columns 4 (lane % 16) .. + 3 (rows past L read as zero).
// Loaded ahead of the epilogue so the loads overlap the work before it.
template <bool BF>
using XRow = typename std::conditional<BF, u32x2, u32x4>::type;
template <bool BF>
__device__ inline void load_rows_x(XRow<BF> (&xw)[8], __amdgpu_buffer_rsrc_t rx, uint32_t mbytes,
                                   int lane) {
  const int sr = lane >> 4, sc = lane & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t o = (uint32_t)(4 * i + sr) * mbytes;
    if constexpr (BF)
      xw[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rx, o + 8 * sc, 0, 0));
    else
      xw[i] = dev_load16(rx, o + 16 * sc);
  }
}

// write_rows for a tensor that went through the fused qk_norm: the staged
// rows are the gradient dy with respect to the normalised rows; with
// g = dy * gain and xh = (x - mean) * rstd (x from load_rows_x) each final
// row becomes dx = rstd * (g - mean(g) - xh * mean(g * xh)). The lane's 4
// columns of dy * xh and dy are summed over the rows it writes and then over
// the wave into part[0 .. 2 kDh) (gain, then bias).
template <bool BF>
__device__ inline void write_rows_qkn(const float* srow, const int32_t* mpos,
                                      const int32_t* mkind, void* final_base, int64_t rs,
                                      const XRow<BF> (&xw)[8], const float* mean,
                                      const float* rstd, const void* gain, float* part,
                                      int lane) {
  using T = typename std::conditional<BF, __bf16, float>::type;
  const int sr = lane >> 4, sc = lane & 15;
  float gn[4], acc_g[4] = {0.f, 0.f, 0.f, 0.f}, acc_b[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 4; ++e) gn[e] = (float)reinterpret_cast<const T*>(gain)[4 * sc + e];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int R = 4 * i + sr;
    const bool live = mkind[R] == 1;  // uniform over the row's 16 lanes
    const f32x4 dy = *reinterpret_cast<const f32x4*>(srow + R * kStageStride + 4 * sc);
    float x[4];
    if constexpr (BF) {
      const u32x2 w = xw[i];
      x[0] = __uint_as_float(w[0] << 16);
      x[1] = __uint_as_float(w[0] & 0xffff0000u);
      x[2] = __uint_as_float(w[1] << 16);
      x[3] = __uint_as_float(w[1] & 0xffff0000u);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(xw[i][e]);
    }
    const float mu = mean[R], rs_ = rstd[R];
    float xh[4], gg[4], sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xh[e] = (x[e] - mu) * rs_;
      gg[e] = dy[e] * gn[e];
      sg += gg[e];
      sgx = fmaf(gg[e], xh[e], sgx);
    }
#pragma unroll
    for (int m = 1; m < 16; m *= 2) {
      sg += __shfl_xor(sg, m);
      sgx += __shfl_xor(sgx, m);
    }
    const float mg = sg * (1.f / kDh), mgx = sgx * (1.f / kDh);
    float dx[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) dx[e] = rs_ * (gg[e] - mg - xh[e] * mgx);
    if (live) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc_g[e] = fmaf(dy[e], xh[e], acc_g[e]);
        acc_b[e] += dy[e];
      }
      T* dst = reinterpret_cast<T*>(final_base) + (int64_t)mpos[R] * rs + 4 * sc;
      if constexpr (BF)
        *reinterpret_cast<u32x2*>(dst) =
            u32x2{dev_pack_bf16(dx[0], dx[1]), dev_pack_bf16(dx[2], dx[3])};
      else
        *reinterpret_cast<f32x4*>(dst) = f32x4{dx[0], dx[1], dx[2], dx[3]};
    }
  }
  // the 4 row groups of the wave hold the same columns: fixed-order sum
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc_g[e] += __shfl_xor(acc_g[e], 16);
    acc_g[e] += __shfl_xor(acc_g[e], 32);
    acc_b[e] += __shfl_xor(acc_b[e], 16);
    acc_b[e] += __shfl_xor(acc_b[e], 32);
  }
  if (sr == 0) {
    *reinterpret_cast<f32x4*>(part + 4 * sc) = f32x4{acc_g[0], acc_g[1], acc_g[2], acc_g[3]};
    *reinterpret_cast<f32x4*>(part + kDh + 4 * sc) =
        f32x4{acc_b[0], acc_b[1], acc_b[2], acc_b[3]};
  }
}

// ---------------------------------------------------------------- short segments

// Segments of at most 32 gathered rows: one wave takes a whole unit, every
// query and key of it at once, and computes all three gradients, so q, k, v,
// dout and out are each read once. D comes from out and dout on the way in.
// S = Q K^T and dP = dout V^T put one key in each lane (the dK/dV kernel's
// layout); dV^T = dout^T P and dK^T = Q^T dS follow as there. dS^T is then
// written to LDS, and dQ^T = K^T dS^T takes both operands from transpose
// reads (K^T of the staged K, dS of the staged dS^T). Rows are written
// through the LDS staging area as 128-byte lines.
// QKN: the module's qk_norm fused in (a.qkn set; one pattern): q and k rows
// are normalised while staged, and the dq, dk rows go through the layer
// norm's backward before they are written; bf16 with qk_norm is held to 168
// VGPRs (3 waves per SIMD), which the early loads of the epilogue's input
// rows would otherwise exceed.
template <bool CAUSAL, bool BF, bool QKN = false>
__global__ __launch_bounds__(64, (QKN && BF) ? 3 : 1) void bwd_short_kernel(const BwdArgs a) {
  using T = typename std::conditional<BF, __bf16, float>::type;
  constexpr int ST = lds_stride<BF>();
  constexpr int kTileBytes = 32 * ST * (int)sizeof(T);
  // Q, dout then dS^T, K; lse2, D; qk_norm row statistics (q mean, q rstd,
  // k mean, k rstd)
  constexpr int kBytes = 3 * kTileBytes + 2 * 32 * 4 + (QKN ? 4 * 32 * 4 : 0);
  static_assert(kTileBytes % 16 == 0, "LDS alignment");
  static_assert(3 * kTileBytes >= kStageBytes, "epilogue staging fits the tiles");
  __shared__ __attribute__((aligned(16))) char smem[kBytes];
  T* const Qs = reinterpret_cast<T*>(smem);
  T* const Ds = reinterpret_cast<T*>(smem + kTileBytes);  // dout, later dS^T
  T* const Ks = reinterpret_cast<T*>(smem + 2 * kTileBytes);
  float* const ls = reinterpret_cast<float*>(smem + 3 * kTileBytes);
  float* const dd = ls + 32;
  float* const qst = dd + 32;  // qk_norm statistics (QKN only)

  UnitTile tl;
  if (!decode_unit_tile<false>(a, blockIdx.x, &tl)) return;
  const UnitGeom g = unit_geom<T>(a, tl);

  const int lane = threadIdx.x;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int64_t rowbase = g.headbase + (g.seg0 + g.off) * g.rs;
  // q, k, v and dq, dk, dv: with qk_norm fused a caller-given position
  // stride (they may interleave in one buffer); out and dout as the output
  const int64_t rsi = QKN ? a.in_rs : g.rs;
  const int64_t headbase_in = QKN ? tl.b * a.N * rsi + (int64_t)tl.h * kDh : g.headbase;
  const int64_t rowbase_in = headbase_in + (g.seg0 + g.off) * rsi;
  const uint32_t mbytes_in = QKN ? (uint32_t)((int64_t)g.r * rsi * (int64_t)sizeof(T)) : g.mbytes;
  const uint32_t range_in =
      QKN ? (uint32_t)(g.L - 1) * mbytes_in + (uint32_t)(kDh * sizeof(T)) : g.range;
  const auto rq = dev_rsrc(reinterpret_cast<const T*>(a.q) + rowbase_in, range_in);
  const auto rk = dev_rsrc(reinterpret_cast<const T*>(a.k) + rowbase_in, range_in);
  const auto rv = dev_rsrc(reinterpret_cast<const T*>(a.v) + rowbase_in, range_in);
  const auto rdo = dev_rsrc(reinterpret_cast<const T*>(a.dout) + rowbase, g.range);
  const auto ro = dev_rsrc(reinterpret_cast<const T*>(a.out) + rowbase, g.range);

  // rows past L load as zeros: D = 0 there, and lse2 = +inf makes P = 0.
  // Pairs with one row stride each: (q, dout) and (k, out), or with qk_norm
  // (q, k) and (dout, out).
  using Stg = PairStager<BF, 32, 64>;
  Stg s1, s2;
  if constexpr (QKN) {
    s1.init(lane, mbytes_in);
    s2.init(lane, g.mbytes);
    s1.load(rq, rk, 0);
    s2.load(rdo, ro, 0);
  } else {
    s1.init(lane, g.mbytes);
    s2.init(lane, g.mbytes);
    s1.load(rq, rdo, 0);
    s2.load(rk, ro, 0);
  }
  RowFrag<BF> vf;  // B operand of dP = dout V^T
  vf.load(rv, (uint32_t)n * mbytes_in, hh);
  int64_t pos = 0;
  float l2 = INFINITY;
  if (n < g.L) {
    pos = g.seg0 + g.off + (int64_t)n * g.r;
    l2 = a.lse[g.bh * a.N + pos] * kLog2e;
  }
  // D: each chunk's share of dout . out, summed over the chunks of its row
  // (lanes with the same lane / kChunksPerRow)
  constexpr int CPR = Stg::kChunksPerRow;
#pragma unroll
  for (int i = 0; i < Stg::CK; ++i) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t o = s2.rb[i][e], d = QKN ? s2.ra[i][e] : s1.rb[i][e];
      if constexpr (BF) {
        s = fmaf(__uint_as_float(o << 16), __uint_as_float(d << 16), s);
        s = fmaf(__uint_as_float(o & 0xffff0000u), __uint_as_float(d & 0xffff0000u), s);
      } else {
        s = fmaf(__uint_as_float(o), __uint_as_float(d), s);
      }
    }
#pragma unroll
    for (int m = 1; m < CPR; m *= 2) s += __shfl_xor(s, m);
    if (lane % CPR == 0) dd[(lane + 64 * i) / CPR] = s;
  }
  if constexpr (QKN) {
    qkn_normalize<BF>(s1.ra, a.qkn[0], a.qkn[1], a.qkn_eps, g.L, lane, qst, qst + 32);
    qkn_normalize<BF>(s1.rb, a.qkn[2], a.qkn[3], a.qkn_eps, g.L, lane, qst + 64, qst + 96);
    s1.store(lane, Qs, Ks);
    s2.store_first(lane, Ds);
  } else {
    s1.store(lane, Qs, Ds);
    s2.store_first(lane, Ks);
  }
  if (hh == 0) ls[n] = l2;
  __syncthreads();

  RowFrag<BF> kf;  // B operand of S = Q K^T
  kf.load_lds(Ks + n * ST, hh);
  f32x16 S, dP;
#pragma unroll
  for (int v = 0; v < 16; ++v) S[v] = dP[v] = 0.f;
  if constexpr (BF) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qs + n * ST + 16 * ks + 8 * hh);
      const bf16x8 da = *reinterpret_cast<const bf16x8*>(Ds + n * ST + 16 * ks + 8 * hh);
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf.x[ks], S, 0, 0, 0);
      dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf.x[ks], dP, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      S = __builtin_amdgcn_mfma_f32_32x32x2f32(Qs[n * ST + 2 * ks + hh], kf.x[ks], S, 0, 0, 0);
      dP = __builtin_amdgcn_mfma_f32_32x32x2f32(Ds[n * ST + 2 * ks + hh], vf.x[ks], dP, 0, 0, 0);
    }
  }
  // register v: query 8(v/4) + 4hh + v%4, key n; causal: the whole unit is
  // the diagonal block
  float pv[16], sv[16];
  const float sl2 = a.sl2;
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    const int qi = 8 * gq + 4 * hh;
    const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + qi);
    const f32x4 d4 = *reinterpret_cast<const f32x4*>(dd + qi);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = 4 * gq + j;
      float p = __builtin_amdgcn_exp2f(fmaf(S[v], sl2, -l4[j]));
      if (CAUSAL && qi + j < n) p = 0.f;
      pv[v] = p;
      sv[v] = p * (dP[v] - d4[j]);
    }
  }

  f32x16 dK[2], dV[2], dQ[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) dK[db][v] = dV[db][v] = dQ[db][v] = 0.f;
  const uint32_t trl = tr_lane_offset<ST>(lane);
  if constexpr (BF) {
    const lds_cptr qbase = (lds_cptr)smem;
    const lds_cptr dbase = qbase + kTileBytes;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8 pb = to_bf16x8(pv + 8 * c);
      const bf16x8 sb = to_bf16x8(sv + 8 * c);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const uint32_t o = trl + (uint32_t)(16 * c * ST + db * 32) * 2;
        dV[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_fragment(dbase, o, ST), pb, dV[db], 0,
                                                         0, 0);
        dK[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_fragment(qbase, o, ST), sb, dK[db], 0,
                                                         0, 0);
      }
    }
  } else {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int qi = 8 * (v >> 2) + 4 * hh + (v & 3);
        dV[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Ds[qi * ST + db * 32 + n], pv[v], dV[db], 0,
                                                      0, 0);
        dK[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Qs[qi * ST + db * 32 + n], sv[v], dK[db], 0,
                                                      0, 0);
      }
  }
  __syncthreads();  // dout consumed: its tile takes dS^T (row = key n)
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    T* dst = Ds + n * ST + 8 * gq + 4 * hh;
    if constexpr (BF) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{dev_pack_bf16(sv[4 * gq], sv[4 * gq + 1]),
                                             dev_pack_bf16(sv[4 * gq + 2], sv[4 * gq + 3])};
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[j] = sv[4 * gq + j];
    }
  }
  __syncthreads();
  // dQ^T[dim][query] += K^T[dim][key] dS^T[key][query]
  if constexpr (BF) {
    const lds_cptr sbase = (lds_cptr)smem + kTileBytes;
    const lds_cptr kbase = (lds_cptr)smem + 2 * kTileBytes;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8 sb = tr_fragment(sbase, trl + (uint32_t)(16 * c * ST) * 2, ST);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const uint32_t o = trl + (uint32_t)(16 * c * ST + db * 32) * 2;
        dQ[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_fragment(kbase, o, ST), sb, dQ[db], 0,
                                                         0, 0);
      }
    }
  } else {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ki = 8 * (v >> 2) + 4 * hh + (v & 3);
        dQ[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[ki * ST + db * 32 + n], Ds[ki * ST + n],
                                                      dQ[db], 0, 0, 0);
      }
  }
  XRow<BF> xq[QKN ? 8 : 1];  // QKN: q's input rows for the dq epilogue
  if constexpr (QKN) load_rows_x<BF>(xq, rq, mbytes_in, lane);
  __syncthreads();  // tiles consumed: the staging area takes their place

  const PatDev& P = a.pat[tl.p];
  const int64_t slots = P.units * P.lmax;
  const int64_t prow0 = (g.bh * P.nseg + tl.seg) * P.lmax;  // the unit's first slot
  float* const srow = reinterpret_cast<float*>(smem);
  int32_t* const mpos = reinterpret_cast<int32_t*>(srow + 32 * kStageStride);
  int32_t* const mkind = mpos + 32;
  if (hh == 0) {
    int32_t kind = 0;
    if (n < g.L) kind = coverage(a, (uint32_t)pos, tl.h) == 1 ? 1 : 2;
    mpos[n] = n < g.L ? (int32_t)pos : -1;  // positions are below 2^31
    mkind[n] = kind;
  }
  T* const part = reinterpret_cast<T*>(a.ws + P.po_off) + prow0 * kDh;
  stage_row(srow, dQ, a.scale, n, hh);
  XRow<BF> xk[QKN ? 8 : 1];  // QKN: k's input rows for the dk epilogue
  if constexpr (QKN) load_rows_x<BF>(xk, rk, mbytes_in, lane);
  __syncthreads();
  if constexpr (QKN) {
    const int64_t unit = prow0 / P.lmax;
    write_rows_qkn<BF>(srow, mpos, mkind, reinterpret_cast<T*>(a.dq) + headbase_in, rsi, xq,
                       qst, qst + 32, a.qkn[0], a.qkn_part + unit * 2 * kDh, lane);
  } else {
    write_rows<BF>(srow, mpos, mkind, reinterpret_cast<T*>(a.dq) + g.headbase, g.rs, part, lane);
  }
  __syncthreads();
  stage_row(srow, dK, a.scale, n, hh);
  __syncthreads();
  if constexpr (QKN) {
    const int64_t unit = prow0 / P.lmax;
    write_rows_qkn<BF>(srow, mpos, mkind, reinterpret_cast<T*>(a.dk) + headbase_in, rsi, xk,
                       qst + 64, qst + 96, a.qkn[2], a.qkn_part + (a.qkn_units + unit) * 2 * kDh,
                       lane);
  } else {
    write_rows<BF>(srow, mpos, mkind, reinterpret_cast<T*>(a.dk) + g.headbase, g.rs,
                   part + slots * kDh, lane);
  }
  __syncthreads();
  stage_row(srow, dV, 1.f, n, hh);
  __syncthreads();
  write_rows<BF>(srow, mpos, mkind, reinterpret_cast<T*>(a.dv) + headbase_in, rsi,
                 part + 2 * slots * kDh, lane);
}

// ---------------------------------------------------------------- row passes

constexpr int kLanesPerRow = 4;
constexpr int kDimsPerLane = kDh / kLanesPerRow;  // 16
constexpr int kRowThreads = 256;
constexpr int kRowsPerBlock = kRowThreads / kLanesPerRow;

// 16 consecutive elements of a row as floats.
template <bool BF>
__device__ inline void load16(const void* base, int64_t elem, float* x) {
  if constexpr (BF) {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(base) + elem);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x4 u = p[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[8 * j + 2 * i] = __uint_as_float(u[i] << 16);
        x[8 * j + 2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      }
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + elem);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 u = p[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * j + i] = u[i];
    }
  }
}

template <bool BF>
__device__ inline void store16(void* base, int64_t elem, const float* x) {
  if constexpr (BF) {
    u32x4* p = reinterpret_cast<u32x4*>(reinterpret_cast<__bf16*>(base) + elem);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      p[j] = u32x4{dev_pack_bf16(x[8 * j], x[8 * j + 1]), dev_pack_bf16(x[8 * j + 2], x[8 * j + 3]),
                   dev_pack_bf16(x[8 * j + 4], x[8 * j + 5]),
                   dev_pack_bf16(x[8 * j + 6], x[8 * j + 7])};
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + elem);
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = f32x4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
  }
}

// D = dout . out per row; 4 lanes per row, 16 dimensions each.
template <bool BF>
__global__ __launch_bounds__(kRowThreads) void bwd_prep_kernel(const BwdRowArgs a,
                                                              const FastDiv h_div) {
  const uint32_t row = blockIdx.x * kRowsPerBlock + (threadIdx.x / kLanesPerRow);
  const int sub = threadIdx.x % kLanesPerRow;
  if (row >= (uint32_t)(a.N * a.H)) return;  // all 4 lanes of a row leave together
  const uint32_t t = fdiv(row, h_div);
  const int32_t h = (int32_t)(row - t * (uint32_t)a.H);
  const int64_t b = blockIdx.y;
  const int64_t elem = ((b * a.N + t) * a.H + h) * kDh + kDimsPerLane * sub;
  float o[kDimsPerLane], d[kDimsPerLane];
  load16<BF>(a.out, elem, o);
  load16<BF>(a.dout, elem, d);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kDimsPerLane; ++i) s = fmaf(o[i], d[i], s);
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  if (sub == 0) a.dvec[(b * a.H + h) * a.N + t] = s;
}

// Sum of the per-pattern partials of rows two or more patterns gather; zero
// gradients for rows no pattern gathers. Rows one pattern gathers were
// written by the dK/dV and dQ kernels (or the short-segment kernel). Every
// covering pattern's partials of all three gradients are loaded before any
// is added, so a row costs one memory round trip rather than one per pattern
// and gradient; instantiated per pattern count.
template <bool BF, int NP>
__global__ __launch_bounds__(kRowThreads) void bwd_merge_kernel(const BwdRowArgs a,
                                                               const FastDiv h_div) {
  const uint32_t row = blockIdx.x * kRowsPerBlock + (threadIdx.x / kLanesPerRow);
  const int sub = threadIdx.x % kLanesPerRow;
  if (row >= (uint32_t)(a.N * a.H)) return;
  const uint32_t t = fdiv(row, h_div);
  const int32_t h = (int32_t)(row - t * (uint32_t)a.H);
  const int64_t b = blockIdx.y;

  int32_t ci[NP];
  int cover = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    ci[i] = (int32_t)compact_index(t, a.pat[i], head_offset(h, a.pat[i].r));
    cover += ci[i] >= 0;
  }
  if (cover == 1) return;

  const int64_t elem = (b * a.N + t) * a.grad_rs + (int64_t)h * kDh + kDimsPerLane * sub;
  void* const dst[3] = {a.dq, a.dk, a.dv};
  // every covering pattern's partials of all three gradients are loaded
  // before any is added (the sum is taken in fp32)
  using Raw = typename std::conditional<BF, u32x4[2], f32x4[4]>::type;
  Raw x[3][NP];
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (ci[i] < 0) continue;
      const PatDev& P = a.pat[i];
      const int64_t slots = P.units * P.lmax;
      const int64_t prow = (b * a.H + h) * P.nseg * P.lmax + ci[i];
      const int64_t e = (w * slots + prow) * kDh + kDimsPerLane * sub;
      if constexpr (BF) {
        const u32x4* p =
            reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(a.ws + P.po_off) + e);
        x[w][i][0] = p[0];
        x[w][i][1] = p[1];
      } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(a.ws + P.po_off + e);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[w][i][j] = p[j];
      }
    }
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    float acc[kDimsPerLane];
#pragma unroll
    for (int e = 0; e < kDimsPerLane; ++e) acc[e] = 0.f;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (ci[i] < 0) continue;
      if constexpr (BF) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            acc[8 * j + 2 * k] += __uint_as_float(x[w][i][j][k] << 16);
            acc[8 * j + 2 * k + 1] += __uint_as_float(x[w][i][j][k] & 0xffff0000u);
          }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[4 * j + k] += x[w][i][j][k];
      }
    }
    store16<BF>(dst[w], elem, acc);
  }
}

template <int NW, bool BF>
hipError_t launch_kv_cfg(const BwdArgs& a, bool causal, int64_t grid, hipStream_t st) {
  const dim3 g((uint32_t)grid), b(NW * 64);
  if (causal)
    hipLaunchKernelGGL((bwd_kv_kernel<NW, true, BF>), g, b, 0, st, a);
  else
    hipLaunchKernelGGL((bwd_kv_kernel<NW, false, BF>), g, b, 0, st, a);
  return hipGetLastError();
}

template <int NW, bool BF>
hipError_t launch_q_cfg(const BwdArgs& a, bool causal, int64_t grid, hipStream_t st) {
  const dim3 g((uint32_t)grid), b(NW * 64);
  if (causal)
    hipLaunchKernelGGL((bwd_q_kernel<NW, true, BF>), g, b, 0, st, a);
  else
    hipLaunchKernelGGL((bwd_q_kernel<NW, false, BF>), g, b, 0, st, a);
  return hipGetLastError();
}

template <bool BF>
hipError_t launch_short_cfg(const BwdArgs& a, bool causal, int64_t grid, hipStream_t st) {
  const dim3 g((uint32_t)grid), b(64);
  if (a.qkn[0]) {
    if (causal)
      hipLaunchKernelGGL((bwd_short_kernel<true, BF, true>), g, b, 0, st, a);
    else
      hipLaunchKernelGGL((bwd_short_kernel<false, BF, true>), g, b, 0, st, a);
  } else if (causal) {
    hipLaunchKernelGGL((bwd_short_kernel<true, BF>), g, b, 0, st, a);
  } else {
    hipLaunchKernelGGL((bwd_short_kernel<false, BF>), g, b, 0, st, a);
  }
  return hipGetLastError();
}

// out[w][grp][c] = sum over units u of group grp (consecutive, in order) of
// in[w][u][c]: the per-unit qk_norm gradient partials folded into at most
// kQknGroups rows per tensor; one block per (group, tensor), a thread per
// column, so every read is a contiguous row.
constexpr int kQknGroups = 1024;
__global__ __launch_bounds__(2 * kDh) void qkn_fold_kernel(const float* in, int64_t units,
                                                           int64_t per_group, int64_t groups,
                                                           float* out) {
  const int64_t grp = blockIdx.x, w = blockIdx.y;
  const int c = threadIdx.x;
  const int64_t u0 = grp * per_group, u1 = min(units, u0 + per_group);
  float s = 0.f;
  for (int64_t u = u0; u < u1; ++u) s += in[(w * units + u) * 2 * kDh + c];
  out[(w * groups + grp) * 2 * kDh + c] = s;
}

dim3 row_grid(const BwdRowArgs& a) {
  const int64_t rows = a.N * a.H;
  return dim3((uint32_t)((rows + kRowsPerBlock - 1) / kRowsPerBlock), (uint32_t)a.B);
}

template <bool BF, int NP = 1>
hipError_t launch_bwd_merge_np(const BwdRowArgs& a, const FastDiv& hd, hipStream_t st) {
  if constexpr (NP < kMaxPat) {
    if (a.np > NP) return launch_bwd_merge_np<BF, NP + 1>(a, hd, st);
  }
  hipLaunchKernelGGL((bwd_merge_kernel<BF, NP>), row_grid(a), dim3(kRowThreads), 0, st, a, hd);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep(const BwdRowArgs& a, bool bf16, hipStream_t st) {
  const FastDiv hd = make_fastdiv((uint32_t)a.H);
  if (bf16)
    hipLaunchKernelGGL(bwd_prep_kernel<true>, row_grid(a), dim3(kRowThreads), 0, st, a, hd);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<false>, row_grid(a), dim3(kRowThreads), 0, st, a, hd);
  return hipGetLastError();
}

hipError_t launch_bwd_kv(const BwdArgs& a, bool bf16, bool causal, int64_t grid, hipStream_t st) {
  return bf16 ? launch_kv_cfg<4, true>(a, causal, grid, st)
              : launch_kv_cfg<4, false>(a, causal, grid, st);
}

hipError_t launch_bwd_q(const BwdArgs& a, bool bf16, bool causal, int64_t grid, hipStream_t st) {
  return bf16 ? launch_q_cfg<4, true>(a, causal, grid, st)
              : launch_q_cfg<4, false>(a, causal, grid, st);
}

int64_t qkn_groups(int64_t units) { return units < kQknGroups ? units : kQknGroups; }

hipError_t launch_qkn_fold(const float* part, int64_t units, float* folded, hipStream_t st) {
  const int64_t groups = qkn_groups(units);
  const int64_t per = (units + groups - 1) / groups;
  hipLaunchKernelGGL(qkn_fold_kernel, dim3((uint32_t)groups, 2), dim3(2 * kDh), 0, st, part,
                     units, per, groups, folded);
  return hipGetLastError();
}

hipError_t launch_bwd_short(const BwdArgs& a, bool bf16, bool causal, int64_t grid,
                            hipStream_t st) {
  return bf16 ? launch_short_cfg<true>(a, causal, grid, st)
              : launch_short_cfg<false>(a, causal, grid, st);
}

hipError_t launch_bwd_merge(const BwdRowArgs& a, bool bf16, hipStream_t st) {
  // one pattern of dilation 1 gathers every row exactly once: no partial to
  // sum and no row to zero
  if (a.np == 1 && a.pat[0].r == 1) return hipSuccess;
  const FastDiv hd = make_fastdiv((uint32_t)a.H);
  return bf16 ? launch_bwd_merge_np<true>(a, hd, st) : launch_bwd_merge_np<false>(a, hd, st);
}

}  // namespace da
