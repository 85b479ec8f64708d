// Parameter blocks of the backward kernels (host and device).
#pragma once

#include "da_common.hpp"

namespace da {

// Backward launch over every tile of every pattern. The tile order is the
// forward's (units dealt to XCDs round-robin, patterns sorted by ntile,
// descending); ntile counts tiles of 32 * NW gathered rows (NW = 4: keys
// for the dK/dV kernel, queries for the dQ kernel; NW = 1: whole units of
// the short-segment kernel).
//
// Partial slots: a pattern with po_off >= 0 keeps, at float offset po_off of
// ws, three blocks of units * lmax rows of kDh floats (dq, dk, dv in that
// order; row index ((b * H + h) * nseg + seg) * lmax + m). Rows that exactly
// one pattern gathers bypass them and are written to dq / dk / dv directly.
struct BwdArgs {
  FastDiv h_div;      // division by H
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const void* out;    // read only by the short-segment kernel (for D)
  const float* lse;   // [B, H, N], natural log, from the forward pass
  const float* dvec;  // [B, H, N], D = dout . out per row
  void* dq;
  void* dk;
  void* dv;
  float* ws;
  int64_t B;
  int64_t N;
  int32_t H;
  int32_t np;
  float sl2;    // softmax scale * log2(e)
  float scale;  // softmax scale
  // qk_norm fused into the short-segment kernel: gain_q, bias_q, gain_k,
  // bias_k (q's dtype), or null; q and k then hold the un-normalised rows
  // and dq, dk receive their gradients. qkn_part: [2 (q, k)][qkn_units][2 *
  // kDh] per-unit partial sums of the gain and bias gradients.
  const void* qkn[4];
  float qkn_eps;
  float* qkn_part;
  int64_t qkn_units;
  // qk_norm fused: elements between consecutive positions of q, k, v and
  // of dq, dk, dv (at least H * Dh; they may interleave); out and dout stay
  // [B, N, H, Dh]
  int64_t in_rs;
  PatDev pat[kMaxPat];
  int64_t unit_start[kMaxPat + 1];
};

// Row-wise passes of the backward (D, and the partial sums): per (batch,
// position, head) row.
struct BwdRowArgs {
  const void* out;
  const void* dout;
  float* dvec;
  void* dq;
  void* dk;
  void* dv;
  const float* ws;
  int64_t B;
  int64_t N;
  int32_t H;
  int32_t np;
  int64_t grad_rs;  // elements between consecutive positions of dq, dk, dv
  PatDev pat[kMaxPat];  // caller's order
};

// qk_norm over rows of kDh values, both tensors in one launch.
struct QkNormArgs {
  const void* xq;
  const void* xk;
  void* yq;        // forward outputs
  void* yk;
  const void* dyq;  // backward inputs
  const void* dyk;
  void* dxq;       // backward outputs
  void* dxk;
  const void* gq;  // gains and biases, kDh values each
  const void* bq;
  const void* gk;
  const void* bk;
  float* partials;  // backward: [2][blocks][2 * kDh]
  float* dparams;   // backward: [2 (q, k)][2 (gain, bias)][kDh]
  int64_t rows;
  float eps;
};

}  // namespace da
