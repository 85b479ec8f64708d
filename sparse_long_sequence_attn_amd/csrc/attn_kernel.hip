// Fused dilated-attention kernel for gfx950 (MI355X).
//
// One workgroup computes one query tile of one (batch, head, segment) of one
// pattern: it gathers the segment's dilated rows (every r-th position from
// the head's offset: LongNet blog, "LongNet's attention allocation
// principle"; "LongNet论文精读" page, "Dilated Attention的工作原理" steps 1-2),
// runs softmax attention over them (step 3) with an online softmax, and
// writes the rows back to their positions (step 4) or, when several
// patterns are mixed, to per-pattern partial buffers for the merge kernel.
//
// Work decomposition (NW waves of 64 lanes per workgroup):
//   * each wave owns 32 query rows (BM = 32 * NW per workgroup);
//   * key/value tiles of BN gathered rows are staged through LDS, double
//     buffered, loaded by the whole workgroup with buffer loads whose
//     hardware range check returns zeros for rows past the segment's last
//     gathered row; K is stored row-major with a 16-byte XOR swizzle, V
//     row-major with padded rows, and the PV operand (4 keys of one head
//     dimension per lane) is fetched with the LDS transpose read;
//   * S^T = K Q^T and O^T += V^T P^T run on MFMA 32x32 blocks. With S^T, a
//     lane holds one query and 16 keys of a block, so the row max is in-lane
//     except for one exchange with the lane 32 apart.
// bf16 inputs use v_mfma_f32_32x32x16_bf16 (P rounded to bf16 for PV) and
// take the row sums over the same rounded values on the matrix cores too
// (v_mfma_f32_16x16x32_bf16 against a 0/1 selector): on the vector ALU the
// sums cost more issue slots than the exponentials' overlap with the MFMAs
// leaves. fp32 inputs use v_mfma_f32_32x32x2_f32 with P kept in fp32.
#include <type_traits>

#include "da_common.hpp"
#include "kernels.hpp"

namespace da {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair, round to nearest even (the hardware convert)
__device__ inline uint32_t pack_bf16_rne(float x, float y) {
  bf16x2 p;
  p[0] = (__bf16)x;
  p[1] = (__bf16)y;
  return __builtin_bit_cast(uint32_t, p);
}
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;

struct Tile {
  int64_t b;
  int64_t seg;
  int32_t h;
  int32_t p;    // index into AttnArgs::pat (sorted order)
  int32_t qt;   // query tile inside the segment
};

// Block id -> tile (see AttnArgs for the order). Returns false for the
// padding blocks of XCDs whose list is shorter than the longest one.
__device__ inline bool decode_tile(const AttnArgs& a, uint32_t id, Tile* t) {
  int32_t p;
  uint32_t unit, rank;
  if (!decode_order(a, id, &p, &unit, &rank)) return false;
  const uint32_t bh = fdiv(unit, a.pat[p].nseg_div);
  t->seg = unit - bh * (uint32_t)a.pat[p].nseg;
  const uint32_t b = fdiv(bh, a.h_div);
  t->h = (int32_t)(bh - b * (uint32_t)a.H);
  t->b = b;
  t->p = p;
  t->qt = (int32_t)((uint32_t)a.pat[p].ntile - 1u - rank);
  return true;
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer over [base, base + bytes): 16-byte loads at 32-bit offsets;
// offsets at or past `bytes` read as zero (gfx9 resource word 3 = 0x00020000).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 with
// the LDS bit): lane i's bytes land at dst + 16 i, whatever its offset;
// offsets at or past the buffer's range write zeros. Device pass only: the
// host pass has no such builtin and would drop the kernel's launch stub.
typedef __attribute__((address_space(3))) char* lds_char_ptr;
__device__ inline void dma_load16(__amdgpu_buffer_rsrc_t r, lds_char_ptr dst, uint32_t off,
                                  uint32_t soff = 0) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, soff, 0, 0);
#endif
}

// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane m supplies 4 consecutive 16-bit elements; view them in lane order as
// a 4 x 16 matrix (rows = lanes 4j..4j+3). Lane i receives column i:
// element j = row j, column i.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;
__device__ inline u32x2 lds_read_tr16(const char __attribute__((address_space(3))) * base,
                                      uint32_t byte_off) {
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(base + byte_off)));
}

// Combine a per-lane value with the lane 32 apart (both halves of a query).
__device__ inline float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool BF, int BN, int NBUF = 2, bool DMA = false>
struct Smem {
  // bf16: K [BN][64] swizzled, V [BN][72] (144-byte rows), or with DMA (tiles
  // written by the loads themselves) V [BN][64] swizzled; fp32: K [BN][65],
  // V [BN][64]
  static constexpr int kVStride = BF && !DMA ? kDh + 8 : kDh;
  static constexpr int kKElems = BF ? BN * kDh : BN * (kDh + 1);
  static constexpr int kVElems = BN * kVStride;
  static constexpr int kElemBytes = BF ? 2 : 4;
  static constexpr int kBytes = NBUF * (kKElems + kVElems) * kElemBytes;
};

// NW waves per workgroup, each owning QB blocks of 32 query rows (so every
// K and V fragment read from LDS feeds QB MFMAs); BN keys per LDS tile.
// 4 waves per SIMD: the bf16 4-wave configuration fits in 128 VGPRs without
// spills (configurations that do not fit keep their natural allocation).
// QKN: the DilatedAttention module's qk_norm applied to q and k as they are
// loaded (one-wave workgroups only): each 64-value row becomes
// (x - mean) / sqrt(var + eps) * gain + bias, statistics in fp32.
template <int NW, int QB, int BN, bool CAUSAL, bool FINAL, bool BF, bool QKN = false>
// (fp32 with qk_norm: 2 waves per SIMD, which its registers need without spills)
__global__ __launch_bounds__(NW * 64, QKN ? (BF ? 3 : 2) : 4) void attn_fwd_kernel(
    const AttnArgs a) {
  static_assert(!QKN || (NW == 1 && QB == 1), "qk_norm is fused into one-wave workgroups only");
  using T = typename std::conditional<BF, __bf16, float>::type;
  // one-wave workgroups serve segments of at most 32 gathered rows (one key
  // tile): a single LDS buffer, so more workgroups fit on a CU
  constexpr int NBUF = NW == 1 ? 1 : 2;
  // bf16 multi-wave tiles go global -> LDS directly (buffer loads with the
  // LDS bit): no staging registers and no LDS stores in the loop
  constexpr bool DMA = BF && NBUF == 2;
  using SM = Smem<BF, BN, NBUF, DMA>;
  constexpr int QW = 32 * QB;  // query rows per wave
  constexpr int BM = QW * NW;  // query rows per workgroup
  constexpr int NT = 64 * NW;
  constexpr int KB = BN / 32;
  static_assert(BN % 32 == 0 && BN <= 128, "key tile");

  // epilogue staging of one-wave workgroups: 32 normalised rows (fp32,
  // 68-float stride for conflict-free 16-byte writes) and per-row position,
  // kind and lse
  constexpr int kStageStride = kDh + 4;
  constexpr int kStageBytes = 32 * kStageStride * 4 + 32 * 12;
  constexpr int kSmemBytes =
      NW == 1 && NW * kStageBytes > SM::kBytes ? NW * kStageBytes : SM::kBytes;
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  T* const Ks = reinterpret_cast<T*>(smem);
  T* const Vs = Ks + NBUF * SM::kKElems;  // the K buffers, then the V buffers

  Tile tl;
  if (!decode_tile(a, blockIdx.x, &tl)) return;
  const PatDev& P = a.pat[tl.p];
  const int32_t r = P.r;
  const int64_t wp = P.wp;
  const int32_t off = head_offset(tl.h, r);
  const int32_t L = rows_gathered(wp, off, r);
  const int32_t q0 = tl.qt * BM;
  if (q0 >= L) return;  // last tile of a head one row shorter than lmax

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;

  const int64_t rs = (int64_t)a.H * kDh;  // elements between consecutive positions
  const int64_t seg0 = tl.seg * wp;
  const int64_t headbase = tl.b * a.N * rs + (int64_t)tl.h * kDh;
  // q, k, v rows: the output's layout, or with qk_norm fused a caller-given
  // position stride (q, k, v may interleave in one buffer)
  const int64_t rsi = QKN ? a.in_rs : rs;
  // gathered row m starts at element rowbase + m * mstride
  const int64_t rowbase =
      tl.b * a.N * rsi + (int64_t)tl.h * kDh + gathered_pos(tl.seg, wp, off, r, 0) * rsi;
  const int64_t mstride = (int64_t)r * rsi;

  const int32_t qend_wg = min(L, q0 + BM);
  const int32_t nkt = CAUSAL ? (qend_wg + BN - 1) / BN : (L + BN - 1) / BN;
  const int32_t qw0 = q0 + wv * QW;
  const int32_t qend_w = min(L, qw0 + QW);
  const int32_t nkt_w = qw0 >= L ? 0 : (CAUSAL ? (qend_w + BN - 1) / BN : nkt);
  // wave-uniform values the key loop tests, held in scalar registers
  const int wvs = __builtin_amdgcn_readfirstlane(wv);
  const int32_t nkt_ws = __builtin_amdgcn_readfirstlane(nkt_w);
  const int32_t kend_s = __builtin_amdgcn_readfirstlane(CAUSAL ? qw0 + QW : L);
  int32_t mq[QB];  // this lane's queries (gathered indices)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) mq[qb] = qw0 + 32 * qb + n;

  // Buffers over this segment's gathered rows: row m at byte m * mbytes.
  // Rows past L fall outside the range and load as zeros (such keys are
  // masked and such queries are never stored). The host keeps these
  // offsets below 2^31.
  constexpr uint32_t kRowBytes = kDh * sizeof(T);
  const uint32_t mbytes = (uint32_t)(mstride * sizeof(T));
  const uint32_t range = (uint32_t)(L - 1) * mbytes + kRowBytes;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(reinterpret_cast<const T*>(a.q) + rowbase, range);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(reinterpret_cast<const T*>(a.k) + rowbase, range);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(reinterpret_cast<const T*>(a.v) + rowbase, range);

  // ---- query fragments (B operand of S^T = K Q^T), kept in registers
  constexpr int QREGS = BF ? 4 : 32;
  typename std::conditional<BF, bf16x8, float>::type qf[QB][QREGS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const uint32_t qoff = (uint32_t)mq[qb] * mbytes;
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qf[qb][ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, qoff + (16 * ks + 8 * hh) * 2));
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const f32x4 x = __builtin_bit_cast(f32x4, buf_load16(rq, qoff + 16 * c));
        qf[qb][2 * c] = hh ? x[1] : x[0];
        qf[qb][2 * c + 1] = hh ? x[3] : x[2];
      }
    }
  }

  if constexpr (QKN) {
    // this lane holds 32 of the row's 64 values, the lane 32 apart the rest
    // (bf16: dims 16 ks + 8 hh + e; fp32: dims 4 c + hh and 4 c + 2 + hh)
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if constexpr (BF) {
        const uint32_t w = __builtin_bit_cast(u32x4, qf[0][i / 8])[(i % 8) / 2];
        x[i] = __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
      } else {
        x[i] = qf[0][i];
      }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) s += x[i];
    const float mu = pair_sum(s) * (1.f / kDh);
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) v = fmaf(x[i] - mu, x[i] - mu, v);
    const float rstd = __builtin_amdgcn_rsqf(pair_sum(v) * (1.f / kDh) + a.qkn_eps);
    if constexpr (BF) {
      const __bf16* gq = reinterpret_cast<const __bf16*>(a.qkn[0]) + 8 * hh;
      const __bf16* bq = reinterpret_cast<const __bf16*>(a.qkn[1]) + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 gw = *reinterpret_cast<const u32x4*>(gq + 16 * ks);
        const u32x4 bw = *reinterpret_cast<const u32x4*>(bq + 16 * ks);
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float y0 = fmaf((x[8 * ks + 2 * j] - mu) * rstd, __uint_as_float(gw[j] << 16),
                                __uint_as_float(bw[j] << 16));
          const float y1 = fmaf((x[8 * ks + 2 * j + 1] - mu) * rstd,
                                __uint_as_float(gw[j] & 0xffff0000u),
                                __uint_as_float(bw[j] & 0xffff0000u));
          o[j] = pack_bf16_rne(y0, y1);
        }
        qf[0][ks] = __builtin_bit_cast(bf16x8, o);
      }
    } else {
      const float* gq = reinterpret_cast<const float*>(a.qkn[0]);
      const float* bq = reinterpret_cast<const float*>(a.qkn[1]);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const f32x4 gw = *reinterpret_cast<const f32x4*>(gq + 4 * c);
        const f32x4 bw = *reinterpret_cast<const f32x4*>(bq + 4 * c);
        qf[0][2 * c] = fmaf((x[2 * c] - mu) * rstd, hh ? gw[1] : gw[0], hh ? bw[1] : bw[0]);
        qf[0][2 * c + 1] =
            fmaf((x[2 * c + 1] - mu) * rstd, hh ? gw[3] : gw[2], hh ? bw[3] : bw[2]);
      }
    }
  }

  // ---- key/value tile staging: global -> registers -> LDS. Thread chunk c
  // of a tile is 16 bytes of row c / (row bytes / 16); K and V share offsets.
  constexpr int kChunksPerRow = kRowBytes / 16;  // 8 (bf16) or 16 (fp32)
  constexpr int CK = BN * kChunksPerRow / NT;     // chunks per thread per tensor
  static_assert(CK >= 1 && BN * kChunksPerRow % NT == 0, "tile too small for the workgroup");
  u32x4 kreg[CK], vreg[CK];
  uint32_t koff[CK];
#pragma unroll
  for (int i = 0; i < CK; ++i) {
    const int c = tid + i * NT;
    koff[i] = (uint32_t)(c / kChunksPerRow) * mbytes + (uint32_t)(c % kChunksPerRow) * 16;
  }
  const uint32_t tile_bytes = (uint32_t)BN * mbytes;

  auto load_tile = [&](int kt) {
    if constexpr (DMA) return;
    const uint32_t base = (uint32_t)kt * tile_bytes;
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      kreg[i] = buf_load16(rk, base + koff[i]);
      vreg[i] = buf_load16(rv, base + koff[i]);
    }
  };

  // DMA: each load instruction fills 1 KiB of a tile, lane i the 16 bytes at
  // i * 16 (measured); so lane i of the wave's instruction j fetches the
  // chunk that belongs at that slot: row R = 8 (DW w + j) + i / 8, slot
  // i % 8, which holds chunk (i % 8) ^ swizzle(R). K uses the swizzle of
  // store_tile, V (row-major, 128-byte rows) XORs the chunk index with 4 on
  // rows with bit 1 set, so the transpose reads of 4 consecutive rows hit
  // 4 distinct quarters of the banks. Rows past L load zeros.
  constexpr int DW = DMA ? BN * kRowBytes / 1024 / NW : 1;  // instructions per wave per tensor
  static_assert(!DMA || (BN * kRowBytes) % (1024 * NW) == 0, "DMA tile split");
  uint32_t dk_off[DW], dv_off[DW];
  if constexpr (DMA) {
#pragma unroll
    for (int j = 0; j < DW; ++j) {
      const int R = 8 * (DW * wv + j) + (lane >> 3), slot = lane & 7;
      dk_off[j] = (uint32_t)R * mbytes + (uint32_t)((slot ^ ((R >> 1) & 7)) * 16);
      dv_off[j] = (uint32_t)R * mbytes + (uint32_t)((slot ^ (((R >> 1) & 1) * 4)) * 16);
    }
  }
  auto dma_tile = [&](int kt, int buf) {
    if constexpr (DMA) {
      // the tile's uniform offset goes in the scalar offset field
      const uint32_t base = (uint32_t)kt * tile_bytes;
      const lds_char_ptr kl = (lds_char_ptr)smem + buf * SM::kKElems * 2;
      const lds_char_ptr vl = (lds_char_ptr)smem + (NBUF * SM::kKElems + buf * SM::kVElems) * 2;
#pragma unroll
      for (int j = 0; j < DW; ++j) {
        dma_load16(rk, kl + (DW * wvs + j) * 1024, dk_off[j], base);
        dma_load16(rv, vl + (DW * wvs + j) * 1024, dv_off[j], base);
      }
    }
  };

  // K rows: 16-byte chunk j of row x goes to slot j ^ ((x >> 1) & 7), so the
  // 16 lanes the LDS serves together (rows x..x+15, one chunk index each)
  // hit 16 distinct 16-byte bank groups of the 256-byte bank window.
  auto store_tile = [&](int buf) {
    if constexpr (DMA) return;
    T* K = Ks + buf * SM::kKElems;
    T* V = Vs + buf * SM::kVElems;
    if constexpr (QKN) {
      // each row's chunks sit in kChunksPerRow consecutive lanes (c % chunks
      // = tid % chunks, since NT is a multiple): statistics over those lanes
      const T* gk = reinterpret_cast<const T*>(a.qkn[2]);
      const T* bk = reinterpret_cast<const T*>(a.qkn[3]);
      constexpr int VPC = BF ? 8 : 4;  // values per chunk
      const int d0 = (tid % kChunksPerRow) * VPC;
#pragma unroll
      for (int i = 0; i < CK; ++i) {
        float x[VPC];
#pragma unroll
        for (int e = 0; e < VPC; ++e) {
          if constexpr (BF)
            x[e] = __uint_as_float((e & 1) ? (kreg[i][e / 2] & 0xffff0000u) : (kreg[i][e / 2] << 16));
          else
            x[e] = __uint_as_float(kreg[i][e]);
        }
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < VPC; ++e) s += x[e];
#pragma unroll
        for (int m = 1; m < kChunksPerRow; m *= 2) s += __shfl_xor(s, m);
        const float mu = s * (1.f / kDh);
        float v = 0.f;
#pragma unroll
        for (int e = 0; e < VPC; ++e) v = fmaf(x[e] - mu, x[e] - mu, v);
#pragma unroll
        for (int m = 1; m < kChunksPerRow; m *= 2) v += __shfl_xor(v, m);
        const float rstd = __builtin_amdgcn_rsqf(v * (1.f / kDh) + a.qkn_eps);
#pragma unroll
        for (int e = 0; e < VPC; ++e)
          x[e] = fmaf((x[e] - mu) * rstd, (float)gk[d0 + e], (float)bk[d0 + e]);
#pragma unroll
        for (int e = 0; e < VPC; ++e) {
          if constexpr (BF) {
            if (e & 1) kreg[i][e / 2] = pack_bf16_rne(x[e - 1], x[e]);
          } else {
            kreg[i][e] = __float_as_uint(x[e]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * NT;
      const int row = c / kChunksPerRow, ch = c % kChunksPerRow;
      if constexpr (BF) {
        *reinterpret_cast<u32x4*>(K + row * kDh + ((ch ^ ((row >> 1) & 7)) << 3)) = kreg[i];
        *reinterpret_cast<u32x4*>(V + row * SM::kVStride + ch * 8) = vreg[i];
      } else {
        float* dst = reinterpret_cast<float*>(K) + row * (kDh + 1) + 4 * ch;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = __uint_as_float(kreg[i][e]);
        *reinterpret_cast<u32x4*>(reinterpret_cast<float*>(V) + row * kDh + 4 * ch) = vreg[i];
      }
    }
  };

  // ---- running state per query block: O^T accumulators (2 blocks of 32
  // dims), row max (log2 domain, identical in both lane halves) and this
  // half's row sum
  f32x16 O[2][QB];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[db][qb][v] = 0.f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }
  const float sl2 = a.sl2;
  const int m16 = lane & 15, g16 = lane >> 4;
  bool started = false;  // a tile has set the running max (wave-uniform)
  // bf16 row sums run on the matrix cores: a 16x16x32 MFMA with this 0/1
  // A operand (lane l holds A[l % 16][8 (l / 16) ..]) and a P fragment as B
  // puts in lane l the row sum of query l % 16 (lanes 0-15), l - 16
  // (16-47) or l - 32 (48-63): rows 0-7 of A take the key groups of the
  // lanes that hold queries 0-15, rows 8-15 those of queries 16-31. The
  // running sum stays in that lane order; sum_lane moves a per-query value
  // (lane n and n + 32 hold query n) into it, own_lane moves the sum back.
  const bf16x8 ksel = ((lane & 15) < 8) == ((g16 & 1) == 0)
                          ? bf16x8{(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                                   (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f}
                          : bf16x8{};
  auto sum_lane = [&](float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return g16 == 1 ? __uint_as_float(r[0]) : g16 == 2 ? __uint_as_float(r[1]) : x;
  };
  auto own_lane = [&](float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return g16 == 1 || g16 == 2 ? __uint_as_float(hh ? r[0] : r[1]) : x;
  };
  int32_t qs_s[QB];      // first query of each of the wave's query blocks
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) qs_s[qb] = __builtin_amdgcn_readfirstlane(qw0 + 32 * qb);

  auto compute = [&](int buf, int kt) {
    const T* K = Ks + buf * SM::kKElems;
    const T* V = Vs + buf * SM::kVElems;
    // key blocks (32 keys) of this tile that some query of the wave sees;
    // later blocks are skipped (their scores stay -inf, their PV is skipped)
    // wave-uniform (scalar registers, so the block branches are scalar);
    // compute() only runs for tiles that start before kend_s
    const int nkb = min(KB, (int)((uint32_t)(kend_s - kt * BN + 31) >> 5));
    f32x16 S[KB][QB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (kb >= nkb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int v = 0; v < 16; ++v) S[kb][qb][v] = -INFINITY;
        continue;
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) S[kb][qb] = f32x16{};
      const int row = kb * 32 + n;
      if constexpr (BF) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
              K + row * kDh + (((2 * ks + hh) ^ ((row >> 1) & 7)) << 3));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            S[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ks], S[kb][qb], 0, 0, 0);
        }
      } else {
        const float* Kr = reinterpret_cast<const float*>(K) + row * (kDh + 1) + hh;
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
          const float kv = Kr[2 * ks];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            S[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv, qf[qb][ks], S[kb][qb], 0, 0, 0);
        }
      }
    }

    // mask: keys after the query (causal) or past the segment's rows. Key
    // and query blocks are 32-aligned, so a causal block is before its query
    // block (no mask), on its diagonal, or after it (all dead).
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (kb >= nkb) continue;
      const int32_t kb0 = kt * BN + kb * 32;
      if (CAUSAL) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int32_t qs = qs_s[qb];
          if (kb0 == qs) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (8 * (v >> 2) + (v & 3) > n - 4 * hh) S[kb][qb][v] = -INFINITY;
          } else if (QB > 1 && kb0 > qs) {  // with one query block nkb excludes these
#pragma unroll
            for (int v = 0; v < 16; ++v) S[kb][qb][v] = -INFINITY;
          }
        }
      } else if (kb0 + 32 > L) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int32_t key = kb0 + 8 * (v >> 2) + 4 * hh + (v & 3);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            if (key >= L) S[kb][qb][v] = -INFINITY;
        }
      }
    }

    // the row max of the tile (log2 domain), both lane halves
    auto tile_max = [&](int qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[kb][qb][v]);
      return pair_max(mx) * sl2;
    };
    if constexpr (!BF) {
      // Lazy rescaling: a row's running max (log2 domain) only moves when the
      // tile raises it by more than 8, so p = 2^(s - m_run) stays below 2^8
      // and most tiles skip rescaling O and l.
      float mt[QB];
      bool grow = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        mt[qb] = tile_max(qb);
        grow = grow || (mt[qb] > m_run[qb] + 8.f);
      }
      if (!started) {
        // first tile: O and l are still zero, only the max is set
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) m_run[qb] = mt[qb];
        started = true;
      } else if (__ballot(grow) != 0) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float m_new = fmaxf(m_run[qb], mt[qb]);
          const float alpha = exp2_fast(m_run[qb] - m_new);
          m_run[qb] = m_new;
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < 2; ++db) O[db][qb] *= alpha;
        }
      }
    }

    if constexpr (BF) {
      // The first tile of a row sets its running max m (log2 domain); later
      // tiles form p = 2^(s sl2 - m) against it without a max of their own
      // (p may exceed 1: fp32 sums and bf16 probabilities carry that
      // exactly as well). Only when some row's sum over the tile reaches
      // 2^32 (or overflows) is the tile redone against max(m, its max), with
      // O and l rescaled first; O then stays far inside the fp32 range (each
      // tile adds less than 2^32 times the largest |v|, a row sees fewer
      // than 2^26 tiles). P is rounded to bf16 once: the same packed
      // registers feed the PV MFMA and the row-sum MFMA.
      if (!started) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) m_run[qb] = tile_max(qb);
        started = true;
      }
      u32x4 pw[QB][2 * KB];
      float lsum[QB];
      auto form_p = [&]() {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
          for (int c = 0; c < 2 * KB; ++c) {
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const float p0 = exp2_fast(fmaf(S[c >> 1][qb][8 * (c & 1) + e], sl2, -m_run[qb]));
              const float p1 = exp2_fast(fmaf(S[c >> 1][qb][8 * (c & 1) + e + 1], sl2, -m_run[qb]));
              bf16x2 pr;
              pr[0] = (__bf16)p0;
              pr[1] = (__bf16)p1;
              pw[qb][c][e >> 1] = __builtin_bit_cast(uint32_t, pr);
            }
          }
          f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 2 * KB; ++c)
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ksel, __builtin_bit_cast(bf16x8, pw[qb][c]), t,
                                                        0, 0, 0);
          lsum[qb] = t[0];
        }
      };
      form_p();
      // A p that overflowed to inf turns the row-sum MFMA's zero-weighted
      // terms into NaN. The test is on the bit pattern (sums are >= 0, and
      // NaN and inf order above 2^32 as integers) because this file is
      // compiled assuming no NaN, which would let a float comparison miss it.
      bool over = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        over = over || __float_as_uint(lsum[qb]) >= __float_as_uint(4294967296.f);
      if (__ballot(over) != 0) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float m_new = fmaxf(m_run[qb], tile_max(qb));
          const float alpha = exp2_fast(m_run[qb] - m_new);
          m_run[qb] = m_new;
          l_run[qb] *= sum_lane(alpha);
#pragma unroll
          for (int db = 0; db < 2; ++db) O[db][qb] *= alpha;
        }
        form_p();
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) l_run[qb] += lsum[qb];
      // A operand of O^T += V^T P^T for (dims db*32.., keys 16c..16c+15):
      // lane (n, hh) needs V[16c + 8h + 4hh + j][db*32 + n], j = 0..3, for
      // h = 0, 1. In 16-lane group g (n = 16(g&1) + i, hh = g>>1) lane m
      // points at row 16c + 8h + 4hh + m/4, dims db*32 + 16(g&1) + 4(m&3)..+3;
      // the transpose read then hands lane i the four keys of dim i.
      const char __attribute__((address_space(3)))* vbase =
          (const char __attribute__((address_space(3)))*)smem +
          (NBUF * SM::kKElems + buf * SM::kVElems) * sizeof(T);
      const uint32_t vlane = (uint32_t)((4 * (g16 >> 1) + (m16 >> 2)) * SM::kVStride +
                                        16 * (g16 & 1) + 4 * (m16 & 3)) * 2;
      if constexpr (DMA) {
        static_assert(KB == 2 && SM::kVStride == kDh, "DMA PV reads: 64-key tiles, 128-byte rows");
        // the 64-byte half db of row 16c + 8h + rr sits at half
        // db ^ ((rr >> 1) & 1) of that row. The reads are written out (all
        // eight fragment pairs of a half, then one wait, in one statement):
        // the compiler's own transpose reads would each wait for the next
        // tile's loads, which write the other buffer. The outputs are
        // early-clobber: no fragment may share a register with the address.
        const uint32_t vswz = (uint32_t)((m16 >> 3) & 1);
        const uint32_t vrow = (uint32_t)reinterpret_cast<uintptr_t>(vbase) + vlane;
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const uint32_t addr = vrow + 64u * ((uint32_t)db ^ vswz);
          u32x2 f[8];  // (lo, hi) for c = 0..3
          asm volatile(
              "ds_read_b64_tr_b16 %0, %8\n\t"
              "ds_read_b64_tr_b16 %1, %8 offset:1024\n\t"
              "ds_read_b64_tr_b16 %2, %8 offset:2048\n\t"
              "ds_read_b64_tr_b16 %3, %8 offset:3072\n\t"
              "ds_read_b64_tr_b16 %4, %8 offset:4096\n\t"
              "ds_read_b64_tr_b16 %5, %8 offset:5120\n\t"
              "ds_read_b64_tr_b16 %6, %8 offset:6144\n\t"
              "ds_read_b64_tr_b16 %7, %8 offset:7168\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]),
                "=&v"(f[6]), "=&v"(f[7])
              : "v"(addr)
              : "memory");
#pragma unroll
          for (int c = 0; c < 2 * KB; ++c) {
            if (c >= 2 * nkb) break;
            const bf16x8 vf =
                __builtin_bit_cast(bf16x8, u32x4{f[2 * c][0], f[2 * c][1], f[2 * c + 1][0],
                                                 f[2 * c + 1][1]});
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              O[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  vf, __builtin_bit_cast(bf16x8, pw[qb][c]), O[db][qb], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int c = 0; c < 2 * KB; ++c) {
          if (c >= 2 * nkb) break;
          const uint32_t o0 = vlane + (uint32_t)((16 * c) * SM::kVStride + db * 32) * 2;
          const u32x2 lo = lds_read_tr16(vbase, o0);
          const u32x2 hi = lds_read_tr16(vbase, o0 + 8 * SM::kVStride * 2);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            O[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                vf, __builtin_bit_cast(bf16x8, pw[qb][c]), O[db][qb], 0, 0, 0);
        }
      }
      }
    } else {
      float pf[QB][KB][16];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            pf[qb][kb][v] = exp2_fast(fmaf(S[kb][qb][v], sl2, -m_run[qb]));
            lsum += pf[qb][kb][v];
          }
        l_run[qb] += lsum;
      }
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kb * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
            const float vv = reinterpret_cast<const float*>(V)[key * kDh + db * 32 + n];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              O[db][qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, pf[qb][kb][v], O[db][qb], 0, 0, 0);
          }
    }
  };

  // ---- main loop over key tiles, double-buffered through LDS
  load_tile(0);
  store_tile(0);
  dma_tile(0, 0);
  // every load issued so far (the query fragments included) completes here:
  // otherwise the loop's first use of the fragments waits on the global
  // loads the loop itself has just issued for the next tile
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (DMA) {
    // unrolled by two so each step's buffer is a compile-time constant: the
    // LDS reads then carry the buffer offset as an immediate
    auto step = [&](auto bufc, int kt) {
      constexpr int buf = decltype(bufc)::value;
      // the other buffer was last read before the previous barrier
      if (kt + 1 < nkt) dma_tile(kt + 1, buf ^ 1);
      if (kt < nkt_ws) compute(buf, kt);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's tile writes have landed
      __syncthreads();
    };
    for (int kt = 0; kt < nkt; kt += 2) {
      step(std::integral_constant<int, 0>{}, kt);
      if (kt + 1 < nkt) step(std::integral_constant<int, 1>{}, kt + 1);
    }
  } else if constexpr (NBUF == 2) {
    for (int kt = 0; kt < nkt; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nkt) load_tile(kt + 1);
      if (kt < nkt_w) compute(buf, kt);
      if (kt + 1 < nkt) store_tile(buf ^ 1);
      __syncthreads();
    }
  } else {
    for (int kt = 0; kt < nkt; ++kt) {
      if (kt > 0) {
        __syncthreads();  // the previous tile is consumed before it is overwritten
        load_tile(kt);
        store_tile(0);
        __syncthreads();
      }
      if (kt < nkt_w) compute(0, kt);
    }
  }

  // ---- epilogue: normalise every valid query row and write it
  float l_tot[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) l_tot[qb] = BF ? own_lane(l_run[qb]) : pair_sum(l_run[qb]);
  T* const orow = reinterpret_cast<T*>(a.out) + headbase;
  float* const lse_row = a.lse + ((int64_t)tl.b * a.H + tl.h) * a.N;
  const int64_t seg_end = seg0 + wp;

  if constexpr (NW == 1) {
    // Segments of at most 32 rows are bound by their writes: the rows go out
    // row-contiguous. Each wave stages its 32 rows (fp32) and their metadata
    // in its own LDS region (the K/V tile is no longer read), then 16 lanes
    // write each row: 128 contiguous bytes of bf16 output (256 of fp32 output
    // or of an fp32 partial), where the MFMA layout would scatter 8-byte
    // pieces of 32 rows per store.
    float* const srow = reinterpret_cast<float*>(smem + wv * kStageBytes);
    int32_t* const mpos = reinterpret_cast<int32_t*>(srow + 32 * kStageStride);
    int32_t* const mkind = mpos + 32;  // 0: no row, 1: final output, 2: partial
    float* const mlse = reinterpret_cast<float*>(mkind + 32);
    const int sr = lane >> 4;  // row within a pass of 4 rows
    const int sc = lane & 15;  // 4-value chunk of the row
    auto store4 = [&](T* dst, const f32x4& x) {
      if constexpr (BF) {
        bf16x2 x0, x1;
        x0[0] = (__bf16)x[0];
        x0[1] = (__bf16)x[1];
        x1[0] = (__bf16)x[2];
        x1[1] = (__bf16)x[3];
        *reinterpret_cast<u32x2*>(dst) =
            u32x2{__builtin_bit_cast(uint32_t, x0), __builtin_bit_cast(uint32_t, x1)};
      } else {
        *reinterpret_cast<f32x4*>(dst) = x;
      }
    };
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      __syncthreads();  // LDS free: tile (or the previous query block's rows) consumed
      const bool valid = mq[qb] < L;
      const float inv = valid ? __builtin_amdgcn_rcpf(l_tot[qb]) : 0.f;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = O[db][qb][4 * g + e] * inv;
          *reinterpret_cast<f32x4*>(srow + n * kStageStride + db * 32 + 8 * g + 4 * hh) = x;
        }
      if (hh == 0) {
        int32_t kind = 0, pos32 = -1;
        if (valid) {
          const int64_t pos = gathered_pos(tl.seg, wp, off, r, mq[qb]);
          pos32 = (int32_t)pos;  // positions are below 2^31
          // a row no other pattern gathers is final here; rows several
          // patterns gather go through the partial buffers and the merge
          kind = 1;
          if constexpr (!FINAL) {
            int cover = 0;
            for (int i = 0; i < a.np; ++i)
              cover += compact_index((uint32_t)pos, a.pat[i], head_offset(tl.h, a.pat[i].r)) >= 0;
            kind = cover == 1 ? 1 : 2;
          }
        }
        mpos[n] = pos32;
        mkind[n] = kind;
        mlse[n] = m_run[qb] + __log2f(l_tot[qb]);
      }
      __syncthreads();
      const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int R = 4 * i + sr;
        const int32_t kind = mkind[R];
        if (kind == 0) continue;
        const int64_t pos = mpos[R];
        const f32x4 x = *reinterpret_cast<const f32x4*>(srow + R * kStageStride + 4 * sc);
        const float lse2 = mlse[R];
        const int32_t m = qw0 + 32 * qb + R;  // gathered index of the row
        if (kind == 1) {
          store4(orow + pos * rs + 4 * sc, x);
          if (sc == 0) lse_row[pos] = lse2 * kLn2;
          if constexpr (FINAL) {
            // one pattern: positions of this segment that the head does not
            // gather (the r-1 after each gathered row and, before the first
            // one, the offset rows) get 0 and -inf here
            for (int j = 1; j < r; ++j) {
              if (pos + j >= seg_end) break;
              store4(orow + (pos + j) * rs + 4 * sc, zero4);
              if (sc == 0) lse_row[pos + j] = -INFINITY;
            }
            if (m == 0)
              for (int j = 0; j < off; ++j) {
                store4(orow + (seg0 + j) * rs + 4 * sc, zero4);
                if (sc == 0) lse_row[seg0 + j] = -INFINITY;
              }
          }
        } else {
          const int64_t prow = (((int64_t)tl.b * a.H + tl.h) * P.nseg + tl.seg) * P.lmax + m;
          *reinterpret_cast<f32x4*>(a.ws + P.po_off + prow * kDh + 4 * sc) = x;
          if (sc == 0) a.ws[P.pl_off + prow] = lse2;
        }
      }
    }
  } else {
    // Long segments are bound by the softmax: rows are written straight from
    // the MFMA layout.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (mq[qb] >= L) continue;
      const float inv = __builtin_amdgcn_rcpf(l_tot[qb]);
      const float lse2 = m_run[qb] + __log2f(l_tot[qb]);
      const int64_t pos = gathered_pos(tl.seg, wp, off, r, mq[qb]);
      // A row that no other pattern gathers is final here and is written to
      // out / lse directly; rows several patterns gather go through the
      // partial buffers and the merge kernel.
      bool direct = FINAL;
      if constexpr (!FINAL) {
        int cover = 0;
        for (int i = 0; i < a.np; ++i)
          cover += compact_index((uint32_t)pos, a.pat[i], head_offset(tl.h, a.pat[i].r)) >= 0;
        direct = cover == 1;
      }
      if (direct) {
        auto put = [&](int64_t t, bool zero) {
          T* dst = orow + t * rs + 4 * hh;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int d = db * 32 + 8 * g;
              if constexpr (BF) {
                bf16x2 x0, x1;
                x0[0] = (__bf16)(zero ? 0.f : O[db][qb][4 * g + 0] * inv);
                x0[1] = (__bf16)(zero ? 0.f : O[db][qb][4 * g + 1] * inv);
                x1[0] = (__bf16)(zero ? 0.f : O[db][qb][4 * g + 2] * inv);
                x1[1] = (__bf16)(zero ? 0.f : O[db][qb][4 * g + 3] * inv);
                *reinterpret_cast<u32x2*>(dst + d) =
                    u32x2{__builtin_bit_cast(uint32_t, x0), __builtin_bit_cast(uint32_t, x1)};
              } else {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = zero ? 0.f : O[db][qb][4 * g + e] * inv;
                *reinterpret_cast<f32x4*>(dst + d) = x;
              }
            }
          if (hh == 0) lse_row[t] = zero ? -INFINITY : lse2 * kLn2;
        };
        put(pos, false);
        if constexpr (FINAL) {
          // one pattern: positions of this segment that the head does not
          // gather get 0 and -inf here
          for (int j = 1; j < r; ++j) {
            if (pos + j >= seg_end) break;
            put(pos + j, true);
          }
          if (mq[qb] == 0)
            for (int j = 0; j < off; ++j) put(seg0 + j, true);
        }
      } else {
        const int64_t prow = (((int64_t)tl.b * a.H + tl.h) * P.nseg + tl.seg) * P.lmax + mq[qb];
        float* po = a.ws + P.po_off + prow * kDh + 4 * hh;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = O[db][qb][4 * g + e] * inv;
            *reinterpret_cast<f32x4*>(po + db * 32 + 8 * g) = x;
          }
        if (hh == 0) a.ws[P.pl_off + prow] = lse2;
      }
    }
  }
}

// ---------------------------------------------------------------- one pass

// Geometry of one covering pattern for a one-pass workgroup (all
// wave-uniform): its gathered key rows in the segment that holds the
// group, and the group's rows as gathered indices j0 + s m of that pattern.
struct OnePat {
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t mbytes;  // bytes between consecutive gathered rows
  int32_t Lp;       // rows the head gathers from the segment
  int32_t j0;       // gathered index of group row 0
  int32_t s;        // L / r: gathered rows between consecutive group rows
  int32_t nkt;      // key tiles the workgroup needs
};

// bf16, kOnePassWaves waves x 32 group rows, 64-key tiles loaded straight into LDS (the
// layouts of attn_fwd_kernel's 4-wave path); the key tiles of all covering
// patterns go through one online softmax, and every row is written final.
template <bool CAUSAL>
// (non-causal: 3 waves per SIMD, which its registers need without spills)
__global__ __launch_bounds__(64 * kOnePassWaves, CAUSAL ? 4 : 3) void attn_onepass_kernel(
    const OnePassArgs a) {
  constexpr int NW = kOnePassWaves, BN = 64, KB = BN / 32, BM = 32 * NW;
  constexpr int DW = BN * 128 / 1024 / NW;
  using T = __bf16;
  using SM = Smem<true, BN, 2, true>;
  __shared__ __attribute__((aligned(16))) char smem[SM::kBytes];

  // ---- block -> (batch, head, window, residue, row block). The L * nblk
  // workgroups of one (batch, head, window), which read the same key rows,
  // run on one XCD; those groups are dealt to the XCDs round-robin.
  const int64_t id = blockIdx.x;
  const int32_t xcd = (int32_t)(id % kXcds);
  const int64_t slot = id / kXcds;
  const int64_t per = (int64_t)a.L * a.nblk;
  const int64_t grp = xcd + kXcds * (slot / per);
  if (grp >= a.B * a.H * a.nwin) return;
  const int32_t mem = (int32_t)(slot % per);
  const int32_t res = mem / a.nblk;
  const int32_t blk = a.nblk - 1 - mem % a.nblk;  // later rows (more keys) first
  const int64_t win = grp % a.nwin;
  const int64_t bh = grp / a.nwin;
  const int32_t h = (int32_t)(bh % a.H);
  const int64_t b = bh / a.H;

  const int64_t w0 = win * a.W;
  const int32_t rho = (int32_t)((res - w0 % a.L + a.L) % a.L);  // t0 - w0
  const int32_t cnt = rho < a.W ? (a.W - rho + a.L - 1) / a.L : 0;
  const int32_t q0 = blk * BM;
  if (q0 >= cnt) return;
  const int64_t t0 = w0 + rho;  // position of group row 0

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int64_t rs = (int64_t)a.H * kDh;
  const int64_t headbase = b * a.N * rs + (int64_t)h * kDh;
  const int32_t qw0 = q0 + 32 * wv;  // this wave's first group row
  const int32_t mq = qw0 + n;        // this lane's row
  const int32_t qend_wg = min(cnt, q0 + BM);
  const int32_t qend_w = min(cnt, qw0 + 32);
  T* const orow = reinterpret_cast<T*>(a.out) + headbase;
  float* const lse_row = a.lse + bh * a.N;

  // ---- covering patterns: those whose head offset matches the group's
  // position inside its segment (the same for every row of the group)
  uint32_t cover = 0;
  for (int p = 0; p < a.np; ++p) {
    const PatDev& P = a.pat[p];
    const int32_t off = head_offset(h, P.r);
    const int64_t u = t0 % P.wp;  // position inside the segment
    if (off < P.wp && u >= off && (u - off) % P.r == 0) cover |= 1u << p;
  }
  if (cover == 0) {
    // no pattern gathers these positions: 0 and -inf
    const int sr = lane >> 4, sc = lane & 15;
    for (int m = qw0 + sr; m < qend_w; m += 4) {
      const int64_t t = t0 + (int64_t)a.L * m;
      *reinterpret_cast<u32x2*>(orow + t * rs + 4 * sc) = u32x2{0u, 0u};
      if (sc == 0) lse_row[t] = -INFINITY;
    }
    return;
  }
  auto make_pat = [&](int p) {
    const PatDev& P = a.pat[p];
    OnePat o;
    const int32_t off = head_offset(h, P.r);
    const int64_t seg0 = t0 - t0 % P.wp;
    o.Lp = rows_gathered(P.wp, off, P.r);
    o.j0 = (int32_t)((t0 - seg0 - off) / P.r);
    o.s = a.L / P.r;
    o.mbytes = (uint32_t)((int64_t)P.r * rs * 2);
    const uint32_t range = (uint32_t)(o.Lp - 1) * o.mbytes + kDh * 2;
    const int64_t base = headbase + (seg0 + off) * rs;
    o.rk = make_rsrc(reinterpret_cast<const T*>(a.k) + base, range);
    o.rv = make_rsrc(reinterpret_cast<const T*>(a.v) + base, range);
    const int32_t kend = CAUSAL ? o.j0 + o.s * (qend_wg - 1) + 1 : o.Lp;
    o.nkt = (kend + BN - 1) / BN;
    return o;
  };
  auto next_pat = [&](int p) {  // next covering pattern after p, or a.np
    const uint32_t rest = p + 1 < 32 ? cover >> (p + 1) : 0u;
    return rest ? p + 1 + __builtin_ctz(rest) : a.np;
  };

  // ---- query fragments: group rows at stride L positions
  const uint32_t qbytes = (uint32_t)((int64_t)a.L * rs * 2);
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(reinterpret_cast<const T*>(a.q) + headbase + t0 * rs,
                (uint32_t)(cnt - 1) * qbytes + kDh * 2);
  bf16x8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = __builtin_bit_cast(bf16x8,
                                buf_load16(rq, (uint32_t)mq * qbytes + (16 * ks + 8 * hh) * 2));

  // ---- key/value tiles straight into LDS (the swizzles of attn_fwd_kernel)
  auto dma_tile = [&](const OnePat& o, int kt, int buf) {
    const uint32_t base = (uint32_t)(kt * BN) * o.mbytes;
    const lds_char_ptr kl = (lds_char_ptr)smem + buf * SM::kKElems * 2;
    const lds_char_ptr vl = (lds_char_ptr)smem + (2 * SM::kKElems + buf * SM::kVElems) * 2;
#pragma unroll
    for (int j = 0; j < DW; ++j) {
      const int R = 8 * (DW * wv + j) + (lane >> 3), sl = lane & 7;
      const uint32_t ro = base + (uint32_t)R * o.mbytes;
      dma_load16(o.rk, kl + (DW * wv + j) * 1024, ro + (uint32_t)((sl ^ ((R >> 1) & 7)) * 16));
      dma_load16(o.rv, vl + (DW * wv + j) * 1024, ro + (uint32_t)((sl ^ (((R >> 1) & 1) * 4)) * 16));
    }
  };

  f32x16 O[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[db][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  bool started = false;  // a tile has set the running max (wave-uniform)
  const float sl2 = a.sl2;
  const int m16 = lane & 15, g16 = lane >> 4;
  const uint32_t vlane = (uint32_t)((4 * (g16 >> 1) + (m16 >> 2)) * kDh + 16 * (g16 & 1) +
                                    4 * (m16 & 3)) * 2;
  const uint32_t vswz = (uint32_t)((m16 >> 3) & 1);

  auto compute = [&](const OnePat& o, int buf, int kt) {
    const T* K = reinterpret_cast<const T*>(smem) + buf * SM::kKElems;
    // the keys some row of the wave sees: up to its last row's gathered
    // index (causal) or the segment's rows
    const int32_t kend = CAUSAL ? o.j0 + o.s * (qend_w - 1) + 1 : o.Lp;
    const int nkb = __builtin_amdgcn_readfirstlane(min(KB, (kend - kt * BN + 31) / 32));
    f32x16 S[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (kb >= nkb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) S[kb][v] = -INFINITY;
        continue;
      }
      S[kb] = f32x16{};
      const int row = kb * 32 + n;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            K + row * kDh + (((2 * ks + hh) ^ ((row >> 1) & 7)) << 3));
        S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], S[kb], 0, 0, 0);
      }
    }
    // mask: causal - key j is seen by row m when j <= j0 + s m (its own
    // position or earlier); non-causal - keys past the segment's rows
    const int32_t thr = o.j0 + o.s * mq;
    const int32_t thr_w = __builtin_amdgcn_readfirstlane(o.j0 + o.s * qw0);  // the wave's lowest
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (kb >= nkb) continue;
      const int32_t kb0 = kt * BN + kb * 32;
      if (CAUSAL ? kb0 + 31 > thr_w : kb0 + 32 > o.Lp) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int32_t key = kb0 + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (CAUSAL ? key > thr : key >= o.Lp) S[kb][v] = -INFINITY;
        }
      }
    }

    // lazy rescale and P exactly as in attn_fwd_kernel
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[kb][v]);
    const float mt = pair_max(mx) * sl2;
    if (!started) {
      m_run = mt;
      started = true;
    } else if (__ballot(mt > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 2; ++db) O[db] *= alpha;
    }
    u32x4 pw[2 * KB];
    float lsum = 0.f;
#pragma unroll
    for (int c = 0; c < 2 * KB; ++c) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = exp2_fast(fmaf(S[c >> 1][8 * (c & 1) + e], sl2, -m_run));
        const float p1 = exp2_fast(fmaf(S[c >> 1][8 * (c & 1) + e + 1], sl2, -m_run));
        bf16x2 pr;
        pr[0] = (__bf16)p0;
        pr[1] = (__bf16)p1;
        pw[c][e >> 1] = __builtin_bit_cast(uint32_t, pr);
        const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, lsum, false);
      }
    }
    l_run += lsum;
    // O^T += V^T P^T, V^T from the transpose reads (one statement per half,
    // as in attn_fwd_kernel)
    const uint32_t vrow = (uint32_t)reinterpret_cast<uintptr_t>(
                              (lds_char_ptr)smem + (2 * SM::kKElems + buf * SM::kVElems) * 2) +
                          vlane;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const uint32_t addr = vrow + 64u * ((uint32_t)db ^ vswz);
      u32x2 f[8];
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8\n\t"
          "ds_read_b64_tr_b16 %1, %8 offset:1024\n\t"
          "ds_read_b64_tr_b16 %2, %8 offset:2048\n\t"
          "ds_read_b64_tr_b16 %3, %8 offset:3072\n\t"
          "ds_read_b64_tr_b16 %4, %8 offset:4096\n\t"
          "ds_read_b64_tr_b16 %5, %8 offset:5120\n\t"
          "ds_read_b64_tr_b16 %6, %8 offset:6144\n\t"
          "ds_read_b64_tr_b16 %7, %8 offset:7168\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]),
            "=&v"(f[6]), "=&v"(f[7])
          : "v"(addr)
          : "memory");
#pragma unroll
      for (int c = 0; c < 2 * KB; ++c) {
        if (c >= 2 * nkb) break;
        const bf16x8 vf = __builtin_bit_cast(
            bf16x8, u32x4{f[2 * c][0], f[2 * c][1], f[2 * c + 1][0], f[2 * c + 1][1]});
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, pw[c]),
                                                        O[db], 0, 0, 0);
      }
    }
  };

  // ---- the key tiles of every covering pattern, double-buffered
  int p = next_pat(-1);
  OnePat cur = make_pat(p);
  int kt = 0, buf = 0;
  dma_tile(cur, 0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (;;) {
    int np_ = p, nkt_ = kt + 1;
    OnePat nxt = cur;
    if (nkt_ >= cur.nkt) {
      np_ = next_pat(p);
      nkt_ = 0;
      if (np_ < a.np) nxt = make_pat(np_);
    }
    const bool more = np_ < a.np;
    if (more) dma_tile(nxt, nkt_, buf ^ 1);  // the other buffer was last read before the barrier
    if (qw0 < cnt) {
      const int32_t kend_w = CAUSAL ? cur.j0 + cur.s * (qend_w - 1) + 1 : cur.Lp;
      if (kt * BN < kend_w) compute(cur, buf, kt);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's tile loads have landed
    __syncthreads();
    if (!more) break;
    p = np_;
    kt = nkt_;
    cur = nxt;
    buf ^= 1;
  }

  // ---- every row is final: out and lse written directly
  if (mq >= cnt) return;
  const float l_tot = pair_sum(l_run);
  const float inv = __builtin_amdgcn_rcpf(l_tot);
  const int64_t t = t0 + (int64_t)a.L * mq;
  T* const dst = orow + t * rs + 4 * hh;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      *reinterpret_cast<u32x2*>(dst + db * 32 + 8 * g) =
          u32x2{pack_bf16_rne(O[db][4 * g] * inv, O[db][4 * g + 1] * inv),
                pack_bf16_rne(O[db][4 * g + 2] * inv, O[db][4 * g + 3] * inv)};
    }
  if (hh == 0) lse_row[t] = (m_run + __log2f(l_tot)) * kLn2;
}

template <int NW, int QB, int BN, bool BF>
hipError_t launch_cfg(const AttnArgs& a, bool causal, bool final_out, int64_t grid,
                      hipStream_t st) {
  dim3 g((uint32_t)grid), b(NW * 64);
  if (causal) {
    if (final_out)
      hipLaunchKernelGGL((attn_fwd_kernel<NW, QB, BN, true, true, BF>), g, b, 0, st, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<NW, QB, BN, true, false, BF>), g, b, 0, st, a);
  } else {
    if (final_out)
      hipLaunchKernelGGL((attn_fwd_kernel<NW, QB, BN, false, true, BF>), g, b, 0, st, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<NW, QB, BN, false, false, BF>), g, b, 0, st, a);
  }
  return hipGetLastError();
}

// Launch shapes: bf16 long segments use 4 waves x 64 query rows with 64-key
// tiles; fp32 (not the MFMA-rate path) 4 waves x 32 rows; segments of at
// most 32 gathered rows use one 32-row wave per workgroup with 32-key tiles.
constexpr int kQbBf16 = 1;

}  // namespace

int attn_tile_rows(bool bf16, int nw) { return nw == 4 ? 32 * nw * (bf16 ? kQbBf16 : 1) : 32; }

hipError_t launch_attention_qkn(const AttnArgs& a, bool bf16, bool causal, int64_t grid,
                                hipStream_t st) {
  const dim3 g((uint32_t)grid), b(64);
  if (bf16) {
    if (causal)
      hipLaunchKernelGGL((attn_fwd_kernel<1, 1, 32, true, true, true, true>), g, b, 0, st, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<1, 1, 32, false, true, true, true>), g, b, 0, st, a);
  } else {
    if (causal)
      hipLaunchKernelGGL((attn_fwd_kernel<1, 1, 32, true, true, false, true>), g, b, 0, st, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<1, 1, 32, false, true, false, true>), g, b, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_onepass(const OnePassArgs& a, bool causal, int64_t grid, hipStream_t st) {
  const dim3 g((uint32_t)grid), b(64 * kOnePassWaves);
  if (causal)
    hipLaunchKernelGGL(attn_onepass_kernel<true>, g, b, 0, st, a);
  else
    hipLaunchKernelGGL(attn_onepass_kernel<false>, g, b, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, bool bf16, int nw, bool causal, bool final_out,
                            int64_t grid, hipStream_t st) {
  if (bf16) {
    if (nw == 4) return launch_cfg<4, kQbBf16, 64, true>(a, causal, final_out, grid, st);
    return launch_cfg<1, 1, 32, true>(a, causal, final_out, grid, st);
  }
  if (nw == 4) return launch_cfg<4, 1, 64, false>(a, causal, final_out, grid, st);
  return launch_cfg<1, 1, 32, false>(a, causal, final_out, grid, st);
}

}  // namespace da
