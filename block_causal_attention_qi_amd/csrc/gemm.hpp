// bf16 MFMA GEMM for the block projections on gfx950, C = A W^T with both
// operands K-contiguous (A [M,K] token rows, W [N,K] in the [out, in] Linear
// layout), fp32 accumulation, and fused epilogues:
//   EPI_F32    C[m][n] = acc (+ bias[n])                      (text projection)
//   EPI_RESID  x[m][n] += gate[row kind][n] * acc             (O-proj, down)
//   EPI_SWIGLU a[m][o] = bf16(SiLU(acc_gate) * acc_up)        (gate/up)
//   EPI_QKV    RoPE on q, k from the row's cos/sin, one bf16 rounding, and a
//              scatter into per-segment Q, K [heads][T][128] and V^T
//              [heads][128][Tp] buffers (text rows -> text K/V, which is the
//              cache slot on a capture pass).
//
// The MFMA is issued "transposed": its A operand is a 16-row slice of W
// (output features) and its B operand a 16-row slice of the activations
// (tokens), so each lane ends up holding 4 CONSECUTIVE output features of one
// token.  That puts every RoPE pair (2k, 2k+1) and every float4 residual
// update inside one lane.
//
// Row-count invariance (the MLX page's row-count hazard in "Text K/V reuse"):
// every output element is produced by the same MFMA instruction over the same
// K order whatever M is and wherever the row sits in its tile, so a row's
// result does not depend on how many rows the pass has.  No split-K, no atomics.
#pragma once

#include "common.hpp"

enum GemmEpi { EPI_F32 = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_QKV = 3 };

struct GemmArgs {
  const u16 *A;
  int lda;
  const u16 *W;
  int ldw;
  int M, N, K;  // N counts W rows (for SWIGLU 2F rows -> F outputs)
  int L_rows;   // rows < L_rows are text rows (modulation row 0, text K/V)
  // EPI_F32
  float *C;
  int ldc;
  const float *bias;
  // EPI_RESID
  float *X;
  int ldx;
  const float *gate;    // gate values of text rows; image rows use gate + gate_img_off
  int gate_img_off;
  // EPI_SWIGLU
  u16 *out;
  int ldo;
  int F;
  // EPI_QKV
  int H;
  const float *cos_t, *sin_t, *cos_i, *sin_i;  // [seg rows][64]
  u16 *q_t, *k_t, *vt_t, *q_i, *k_i, *vt_i;
  int seg_t, seg_i;  // text / image segment lengths (rows of Q, K per head)
  int ldv_t, ldv_i;  // V^T row strides (segment length rounded up to 64)
};

namespace gemm {
constexpr int BM = 128;  // tokens per tile
constexpr int BN = 128;  // W rows per tile
constexpr int BK = 64;
constexpr int THREADS = 256;
}  // namespace gemm

// LDS tile: rows of 64 bf16 = 8 chunks of 16 bytes; chunk c of row r is stored
// at slot c ^ (r & 7), so the 16 rows an MFMA operand read touches at one
// chunk index fall on 8 distinct 16-byte bank groups.
QI_DEV int lds_slot(int r, int c) { return r * 8 + (c ^ (r & 7)); }

template <int EPI>
__global__ __launch_bounds__(gemm::THREADS, 2) void gemm_bf16_kernel(const GemmArgs g) {
  using namespace gemm;
  __shared__ u32x4 sA[2][BM * 8];
  __shared__ u32x4 sW[2][BN * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;  // 2 x 2 waves; each 64 tokens x 64 W rows
  const int m0 = blockIdx.x * BM;
  const int tn = blockIdx.y;

  const u16 *pa[4], *pw[4];
  int slot[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + THREADS * j;
    const int row = i >> 3, c = i & 7;
    slot[j] = lds_slot(row, c);
    const int am = min(m0 + row, g.M - 1);  // rows past M load a valid row; never stored
    pa[j] = g.A + (size_t)am * g.lda + c * 8;
    int wr;
    if constexpr (EPI == EPI_SWIGLU) {
      // 16-row slices alternate gate / up for the same 16 outputs
      const int s = row >> 4;
      wr = tn * (BN / 2) + (s >> 1) * 16 + (row & 15) + (s & 1) * g.F;
    } else {
      wr = tn * BN + row;
    }
    pw[j] = g.W + (size_t)wr * g.ldw + c * 8;
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[4], rw[4];
  const int nk = g.K / BK;

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ra[j] = *(const u32x4 *)(pa[j]);
    rw[j] = *(const u32x4 *)(pw[j]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sA[0][slot[j]] = ra[j];
    sW[0][slot[j]] = rw[j];
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int b = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = (kt + 1) * BK;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ra[j] = *(const u32x4 *)(pa[j] + k0);
        rw[j] = *(const u32x4 *)(pw[j] + k0);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + (lane >> 4);
      u32x4 af[4], bt[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) af[f] = sW[b][lds_slot(wn * 64 + f * 16 + (lane & 15), ch)];
#pragma unroll
      for (int t = 0; t < 4; ++t) bt[t] = sA[b][lds_slot(wm * 64 + t * 16 + (lane & 15), ch)];
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[f][t] = mfma16x16x32(af[f], bt[t], acc[f][t]);
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sA[b ^ 1][slot[j]] = ra[j];
        sW[b ^ 1][slot[j]] = rw[j];
      }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  const int g4 = 4 * (lane >> 4);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int m = m0 + wm * 64 + t * 16 + (lane & 15);
    if (m >= g.M) continue;
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const f32x4 gt = acc[2 * p][t], up = acc[2 * p + 1][t];
        const int o = tn * (BN / 2) + wn * 32 + p * 16 + g4;
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = gt[r] / (1.f + __expf(-gt[r])) * up[r];
        u32x2 pk = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        *(u32x2 *)(g.out + (size_t)m * g.ldo + o) = pk;
      }
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int n = tn * BN + wn * 64 + f * 16 + g4;
        const f32x4 v = acc[f][t];
        if constexpr (EPI == EPI_F32) {
          f32x4 o = v;
          if (g.bias) o += *(const f32x4 *)(g.bias + n);
          *(f32x4 *)(g.C + (size_t)m * g.ldc + n) = o;
        } else if constexpr (EPI == EPI_RESID) {
          const float *gp = g.gate + (m < g.L_rows ? 0 : g.gate_img_off) + n;
          f32x4 *xp = (f32x4 *)(g.X + (size_t)m * g.ldx + n);
          *xp = *xp + *(const f32x4 *)gp * v;
        } else {  // EPI_QKV
          const int sec = n / g.H;
          const int w = n - sec * g.H;
          const int head = w >> 7, dh = w & 127;
          const bool txt = m < g.L_rows;
          const int row = txt ? m : m - g.L_rows;
          if (sec < 2) {
            const float *cp = (txt ? g.cos_t : g.cos_i) + (size_t)row * 64 + (dh >> 1);
            const float *sp = (txt ? g.sin_t : g.sin_i) + (size_t)row * 64 + (dh >> 1);
            const float c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
            const float y0 = v[0] * c0 - v[1] * s0, y1 = v[0] * s0 + v[1] * c0;
            const float y2 = v[2] * c1 - v[3] * s1, y3 = v[2] * s1 + v[3] * c1;
            u16 *dst = sec == 0 ? (txt ? g.q_t : g.q_i) : (txt ? g.k_t : g.k_i);
            const int seg = txt ? g.seg_t : g.seg_i;
            u32x2 pk = {pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
            *(u32x2 *)(dst + ((size_t)head * seg + row) * 128 + dh) = pk;
          } else {
            u16 *vt = txt ? g.vt_t : g.vt_i;
            const int ldv = txt ? g.ldv_t : g.ldv_i;
            u16 *base = vt + ((size_t)head * 128 + dh) * ldv + row;
#pragma unroll
            for (int r = 0; r < 4; ++r) base[(size_t)r * ldv] = f32_to_bf16(v[r]);
          }
        }
      }
    }
  }
}
