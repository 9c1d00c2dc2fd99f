// bf16 MFMA GEMM for the block projections on gfx950, C = A W^T with both
// operands K-contiguous (A [M,K] token rows, W [N,K] in the [out, in] Linear
// layout), fp32 accumulation, and fused epilogues:
//   EPI_F32    C[m][n] = acc (+ bias[n])                      (text projection)
//   EPI_RESID  x[m][n] += gate[row kind][n] * acc             (O-proj, down);
//              split over K (small images): chunk s of K writes
//              its fp32 partial sums, and resid_reduce_kernel adds the
//              chunks in order into x
//   EPI_SWIGLU a[m][o] = bf16(SiLU(acc_gate) * acc_up)        (gate/up)
//   EPI_QKV    RoPE on q, k from the row's cos/sin, one bf16 rounding, and a
//              scatter into per-segment Q, K [heads][T][128] and V^T
//              [heads][128][Tp] buffers (text rows -> text K/V, which is the
//              cache slot on a capture pass).
//
// The MFMA (32x32x16 bf16, or 16x16x32 bf16 in the 256 x 256 kernel; both
// give the same fp32 results bit for bit on gfx950) is issued "transposed":
// its A operand is a slice of W rows (output features) and its B operand a
// slice of activation rows (tokens), so each lane ends up holding groups of 4
// CONSECUTIVE output features of one token.  That puts every RoPE pair
// (2k, 2k+1) and every float4 residual update inside one lane.
//
// Row-count invariance (the MLX page's row-count hazard in "Text K/V reuse"):
// every output element is produced by MFMAs over the same K order, with the
// same fp32 result, whatever M is, whichever tile shape the launcher picks and
// wherever the row sits in its tile, and the epilogues round without fused
// multiply-adds, so a row's result does not depend on how many rows the pass
// has.  No atomics.  The
// residual GEMMs of a small image (few rows, too few tiles for the chip) are
// split over K; the split is chosen from the image's token count N alone, so
// the joint and the image-only passes of one render (and both CFG branches)
// take the same chunks and reduce them in the same order.
#pragma once

#include <type_traits>

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
  int batch;         // image rows form `batch` branches of seg_i rows each (true CFG: 2),
                     // each with its own Q, K [heads][seg_i][128] and V^T [heads][128][ldv_i]
  const int *skip;   // first-block cache: when non-NULL and *skip, the launch does nothing
  // EPI_RESID split over K (ksplit > 1): grid = tiles x
  // ksplit; chunk s covers K columns [s K/ksplit, (s+1) K/ksplit) and writes
  // its fp32 partial sums to part + s * M * N ([M][N] row-major)
  int ksplit;
  float *part;
};

namespace gemm {
constexpr int BK = 64;
constexpr int THREADS = 256;  // 4 waves as 2 x 2; each owns (BM/2) tokens x (BN/2) W rows
}  // namespace gemm

// LDS tile: rows of 64 bf16 = 8 chunks of 16 bytes.  gfx950's LDS has 64
// banks (256 bytes), so two consecutive rows share one bank line and a
// ds_read_b128 serves 16 lanes per pass.  Chunk c of row r is stored at slot
// c ^ ((r >> 1) & 7): the 16 consecutive rows one pass reads at a fixed chunk
// index land on 16 distinct 16-byte bank groups, and so do the two rows one
// pass of the tile writes.
QI_DEV int lds_slot(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// Workgroup -> output tile.  Workgroups are handed to the 8 XCDs round-robin
// (id % 8), each XCD with its own L2.  The tile grid is cut into 8 equal
// regions, XM bands of token tiles by 8/XM bands of W-tile columns, one per
// XCD, and each XCD walks its region in groups of 4 token tiles, columns
// fastest, so the tiles that run together share both operands' K slices.
// Wide outputs (32 or more W-tile columns) keep whole token bands (XM = 1: a
// W tile is fetched into one L2 only); narrow ones (16 columns: O-proj and
// down) take 4 x 2 or 2 x 4 regions, so an XCD's 32 concurrent tiles read 4
// token slices and 8 W slices per K step instead of 16 and 2.
QI_DEV void tile_of(int bid, int nTM, int nTN, int &tm, int &tn) {
  int XM = 0;
  if (nTN % 8 == 0 && nTN >= 32) XM = 1;
  else if (nTM % 4 == 0 && nTN % 2 == 0) XM = 4;
  else if (nTM % 2 == 0 && nTN % 4 == 0) XM = 2;
  else if (nTN % 8 == 0) XM = 1;
  if (XM) {
    constexpr int GM = 4;
    const int XN = 8 / XM, RM = nTM / XM, RN = nTN / XN;
    const int xcd = bid & 7, j = bid >> 3;
    const int g = j / (GM * RN), w = j % (GM * RN);
    const int rows = min(GM, RM - g * GM);
    tm = (xcd / XN) * RM + g * GM + w % rows;
    tn = (xcd % XN) * RN + w / rows;
  } else {
    tm = bid % nTM;
    tn = bid / nTM;
  }
}

// ---------------------------------------------------------------- epilogue
// Epilogue arithmetic with every product rounded on its own: contraction into
// fused multiply-adds is switched off for the operators written in these
// bodies, so the compiler cannot fuse them one way in one kernel instance and
// another way in the next (it did: two instances of the same RoPE expression
// differed in one rounding).  Every tile shape, and the joint and image-only
// passes, then round a row's outputs identically.  (HIP's *_rn helpers do not
// give this: once inlined they are contractible.)
// x + gate * v, per component
QI_DEV f32x4 gated_add(f32x4 x, f32x4 gate, f32x4 v) {
#pragma clang fp contract(off)
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = x[i] + gate[i] * v[i];
  return r;
}
// The RoPE rotation of the pair (a, b) by the angle with cosine c and sine s:
// (a c - b s, a s + b c).
QI_DEV float2 rope_pair(float a, float b, float c, float s) {
#pragma clang fp contract(off)
  return float2{a * c - b * s, a * s + b * c};
}

// The 4 consecutive outputs n..n+3 of token m (accumulators v).
template <int EPI>
QI_DEV void store4(const GemmArgs &g, int m, int n, f32x4 v) {
  if constexpr (EPI == EPI_F32) {
    f32x4 o = v;
    if (g.bias) o += *(const f32x4 *)(g.bias + n);
    *(f32x4 *)(g.C + (size_t)m * g.ldc + n) = o;
  } else if constexpr (EPI == EPI_RESID) {
    const float *gp = g.gate + (m < g.L_rows ? 0 : g.gate_img_off) + n;
    f32x4 *xp = (f32x4 *)(g.X + (size_t)m * g.ldx + n);
    *xp = gated_add(*xp, *(const f32x4 *)gp, v);
  }
}

// The LDS a workgroup tile leaves free once its K loop is done, as NOBJ
// objects of SLOTS 16-byte slots each (32 KB or 16 KB), addressed by object so
// that the kernels can keep their operand stages in separate LDS objects.
template <int NOBJ, int SLOTS = 2048>
struct LdsObjs {
  static_assert(NOBJ == 2 || NOBJ == 4, "two or four objects");
  static_assert(SLOTS == 2048 || SLOTS == 1024, "32 KB or 16 KB objects");
  static constexpr int kSlots = SLOTS;
  static constexpr int kRows = SLOTS / 16;  // staged RoPE table rows per object
  u32x4 *p0, *p1, *p2, *p3;
  QI_DEV u32x4 *o(int i) const { return i == 0 ? p0 : i == 1 ? p1 : i == 2 ? p2 : p3; }
};

// RoPE rows of a QKV tile, staged in LDS once the K loop is done (the operand
// buffers are free then).  Each lane rotates 32 pairs of each of its tokens,
// and 32 lanes hold 32 different tokens: read straight from the tables, every
// load instruction would touch 32 rows, which the vector cache serves one row
// at a time.  Staged, the tables are read in whole contiguous rows instead.
// Layout: tile rows come in blocks of R = kRows (128 rows per 32 KB object,
// 64 per 16 KB object; one object per block and table: cos in objects
// 0 .. BM/R - 1, sin in the next BM/R); the float2 (pairs 2q, 2q+1) of row r
// sits at slot (r % R) * 32 + (q ^ (r & 31)) of its object, so the 32 rows
// one half-wave reads at a fixed q hit 32 distinct bank pairs.  A 16-byte
// chunk k (q = 2k, 2k + 1) of the table row lands at the even slot
// (2k) ^ (r & 30), its halves swapped when r is odd.
// The RoPE rows of a tile's BM tokens, loaded from global memory into
// registers (load) and then written to LDS (store), so that a kernel can
// issue the loads before the barrier that frees the LDS.
template <int BM, int THREADS>
struct RopeRows {
  static_assert((BM * 16) % THREADS == 0, "whole passes over the tile's rows");
  static constexpr int IT = BM * 16 / THREADS;  // 16-byte chunks per thread and table
  u32x4 c[IT], s[IT];
  QI_DEV void load(const GemmArgs &g, int m0, int tid) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = tid + THREADS * it;
      const int r = i >> 4, k = i & 15;
      const int m = m0 + r;
      if (m >= g.M) continue;
      const bool txt = m < g.L_rows;
      const size_t off = (size_t)(txt ? m : m - g.L_rows) * 64 + 4 * k;
      c[it] = *(const u32x4 *)((txt ? g.cos_t : g.cos_i) + off);
      s[it] = *(const u32x4 *)((txt ? g.sin_t : g.sin_i) + off);
    }
  }
  template <int NOBJ, int SLOTS>
  QI_DEV void store(const GemmArgs &g, int m0, const LdsObjs<NOBJ, SLOTS> lo, int tid) const {
    constexpr int R = LdsObjs<NOBJ, SLOTS>::kRows;
    static_assert(NOBJ >= 2 * (BM / R) && BM % R == 0, "a cos and a sin object per R rows");
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = tid + THREADS * it;
      const int r = i >> 4, k = i & 15;
      if (m0 + r >= g.M) continue;
      u32x4 cv = c[it], sv = s[it];
      if (r & 1) {
        cv = u32x4{cv[2], cv[3], cv[0], cv[1]};
        sv = u32x4{sv[2], sv[3], sv[0], sv[1]};
      }
      const int chunk = (r % R) * 16 + (k ^ ((r & 30) >> 1));
      lo.o(r / R)[chunk] = cv;
      lo.o(BM / R + r / R)[chunk] = sv;
    }
  }
};

template <int BM, int THREADS, int NOBJ, int SLOTS>
QI_DEV void stage_rope_rows(const GemmArgs &g, int m0, const LdsObjs<NOBJ, SLOTS> lo, int tid) {
  RopeRows<BM, THREADS> rows;
  rows.load(g, m0, tid);
  rows.store(g, m0, lo, tid);
}

// The V section of a QKV wave tile: FS blocks of 32 W rows starting at n0
// (one head, n0 % 64 == 0) and TS blocks of 32 tokens starting at mbase,
// stored transposed into V^T [heads][128][ldv].  For one output feature the
// 32 lanes of a half-wave hold 32 consecutive tokens, so each store writes
// 64 contiguous bytes.
template <int TS, int FS>
QI_DEV void store_v_wave(const GemmArgs &g, int mbase, int n0, const f32x16 (&acc)[FS][TS], int lane) {
  const int w0 = n0 - 2 * g.H;
  const int head = w0 >> 7, dh0 = w0 & 127;
  const int h4 = 4 * (lane >> 5), fr = lane & 31;
#pragma unroll
  for (int t = 0; t < TS; ++t) {
    const int m = mbase + 32 * t + fr;
    if (m >= g.M) continue;
    const bool txt = m < g.L_rows;
    const int row = txt ? m : m - g.L_rows;
    const int br = (txt || g.batch <= 1) ? 0 : row / g.seg_i;  // branch of an image row
    const int brow = row - br * g.seg_i;
    const int ldv = txt ? g.ldv_t : g.ldv_i;
    u16 *base = (txt ? g.vt_t : g.vt_i) + (size_t)br * g.H * ldv + ((size_t)head * 128 + dh0 + h4) * ldv + brow;
#pragma unroll
    for (int f = 0; f < FS; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) base[(size_t)(32 * f + 8 * j + r) * ldv] = f32_to_bf16(acc[f][t][4 * j + r]);
  }
}

// The QKV epilogue of a BM-token workgroup tile whose W rows start at n_tile
// (the section is uniform over the tile: H is a multiple of the tile width).
// Wave (wrow / WT, n0) holds WT = 32 TS tokens x 64 W rows, half of one q or
// k head, as 4 consecutive features of one token per lane and register quad.
// Stored straight from there, every store instruction would touch 32 token
// rows; so the q / k tiles go through LDS twice once the K loop is done:
//   1. the RoPE rows of the tile's tokens are staged (stage_rope_rows), each
//      lane rotates its pairs and rounds them once to bf16;
//   2. each wave writes its 128-byte token half-rows to its own LDS region
//      and reads them back as 16-byte chunks, 8 lanes per token, so a store
//      instruction writes 8 whole half-rows of Q or K [heads][T][128].
// Region layout: 8-byte slot s (features 4 s .. 4 s + 3) of wave row rr sits
// at rr * 16 + (s ^ ((rr >> 1) & 15)): the 32 rows a half-wave writes at a
// fixed s cover all 64 banks, and a 16-byte read of slots 2k, 2k + 1 stays
// one aligned chunk (halves swapped when the XOR term is odd).
template <int BM, int THREADS, int TS, int FS, int NOBJ, int SLOTS>
QI_DEV void qkv_epilogue(const GemmArgs &g, int m0, int n_tile, int wrow, int n0, const f32x16 (&acc)[FS][TS],
                         int tid, const LdsObjs<NOBJ, SLOTS> lo) {
  static_assert(FS == 2, "a wave tile is half a head: 64 W rows");
  constexpr int R = LdsObjs<NOBJ, SLOTS>::kRows;
  constexpr int WT = 32 * TS;
  constexpr int RS = WT * 8;          // 16-byte slots of one wave's region
  constexpr int RPO = SLOTS / RS;     // regions per object
  static_assert(RPO >= 1 && (THREADS / 64) <= RPO * NOBJ, "the waves' regions fit in the objects");
  const int lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 31, hf = lane >> 5;
  if (n_tile / g.H >= 2) {
    store_v_wave<TS, FS>(g, m0 + wrow, n0, acc, lane);
    return;
  }
  const int sec = n0 / g.H;
  const int w0 = n0 - sec * g.H;
  const int head = w0 >> 7, dh0 = w0 & 127;
  __syncthreads();
  stage_rope_rows<BM, THREADS>(g, m0, lo, tid);
  __syncthreads();
  // outputs dh0 + 32 f + 8 j + 4 hf + 0..3 are RoPE pairs 2q, 2q + 1 with
  // q = dh0 / 4 + hf + 8 f + 2 j
  const int q0 = (dh0 >> 2) + hf;
  u32x2 y[TS][FS][4];
#pragma unroll
  for (int t = 0; t < TS; ++t) {
    const int r = wrow + 32 * t + fr;
    const u32x2 *cl2 = (const u32x2 *)lo.o(r / R), *sl2 = (const u32x2 *)lo.o(BM / R + r / R);
#pragma unroll
    for (int f = 0; f < FS; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int slot = (r % R) * 32 + ((q0 + 8 * f + 2 * j) ^ (r & 31));
        const float2 cs = __builtin_bit_cast(float2, cl2[slot]);
        const float2 sn = __builtin_bit_cast(float2, sl2[slot]);
        const f32x4 v = quad(acc[f][t], j);
        const float2 y01 = rope_pair(v[0], v[1], cs.x, sn.x), y23 = rope_pair(v[2], v[3], cs.y, sn.y);
        y[t][f][j] = u32x2{pack_bf16x2(y01.x, y01.y), pack_bf16x2(y23.x, y23.y)};
      }
  }
  __syncthreads();  // every wave is done with the staged tables
  u32x4 *reg = lo.o(wave / RPO) + (wave % RPO) * RS;
  u32x2 *reg2 = (u32x2 *)reg;
#pragma unroll
  for (int t = 0; t < TS; ++t) {
    const int rr = 32 * t + fr;
#pragma unroll
    for (int f = 0; f < FS; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) reg2[rr * 16 + ((8 * f + 2 * j + hf) ^ ((rr >> 1) & 15))] = y[t][f][j];
  }
  __syncthreads();
  u16 *qk_t = sec == 0 ? g.q_t : g.k_t, *qk_i = sec == 0 ? g.q_i : g.k_i;
#pragma unroll
  for (int it = 0; it < WT * 8 / 64; ++it) {
    const int i = lane + 64 * it;
    const int rr = i >> 3, k = i & 7, x = (rr >> 1) & 15;
    u32x4 v = reg[rr * 8 + (k ^ (x >> 1))];
    if (x & 1) v = u32x4{v[2], v[3], v[0], v[1]};
    const int m = m0 + wrow + rr;
    if (m >= g.M) continue;
    const bool txt = m < g.L_rows;
    const int row = txt ? m : m - g.L_rows;
    const int br = (txt || g.batch <= 1) ? 0 : row / g.seg_i;  // branch of an image row
    const int brow = row - br * g.seg_i;
    u16 *dst = (txt ? qk_t : qk_i) + (size_t)br * g.H * g.seg_i +
               ((size_t)head * (txt ? g.seg_t : g.seg_i) + brow) * 128 + dh0 + 8 * k;
    *(u32x4 *)dst = v;
  }
}

// SwiGLU outputs o..o+3 of token m from the gate and up accumulators.  The
// sigmoid's reciprocal is v_rcp_f32 (within 1 ulp; the output is rounded to
// bf16 next), not the ten-instruction IEEE division sequence.
QI_DEV void store4_swiglu(const GemmArgs &g, int m, int o, f32x4 gt, f32x4 up) {
  float y[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) y[r] = gt[r] * __builtin_amdgcn_rcpf(1.f + __expf(-gt[r])) * up[r];
  *(u32x2 *)(g.out + (size_t)m * g.ldo + o) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
}

template <int EPI, int BM, int BN>
__global__ __launch_bounds__(gemm::THREADS, (BM * BN >= 256 * 256) ? 1 : 2) void gemm_bf16_kernel(const GemmArgs g) {
  using namespace gemm;
  if (g.skip && *g.skip) return;
  constexpr int WT = BM / 2, WF = BN / 2;    // per-wave tokens, W rows
  constexpr int TS = WT / 32, FS = WF / 32;  // 32-row subtiles per wave
  constexpr int CA = BM * 8 / THREADS, CW = BN * 8 / THREADS;  // 16-byte chunks per thread
  static_assert(FS % 2 == 0, "SwiGLU pairs gate/up subtiles inside a wave");
  __shared__ u32x4 sA[2][BM * 8];
  __shared__ u32x4 sW[2][BN * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int nTM = (g.M + BM - 1) / BM;
  const int nTN = (EPI == EPI_SWIGLU ? g.F / (BN / 2) : g.N / BN);
  // split over K (EPI_RESID only): the workgroup's chunk and its K columns
  const bool split = EPI == EPI_RESID && g.ksplit > 1;
  const int ntile = nTM * nTN;
  const int kchunk = split ? (int)(blockIdx.x / ntile) : 0;
  const int kc = split ? g.K / g.ksplit : g.K;
  int tm, tn;
  tile_of(split ? (int)(blockIdx.x % ntile) : (int)blockIdx.x, nTM, nTN, tm, tn);
  const int m0 = tm * BM;

  const u16 *pa[CA], *pw[CW];
  int slot_a[CA], slot_w[CW];
#pragma unroll
  for (int j = 0; j < CA; ++j) {
    const int i = tid + THREADS * j;
    const int row = i >> 3, c = i & 7;
    slot_a[j] = lds_slot(row, c);
    const int am = min(m0 + row, g.M - 1);  // rows past M load a valid row; never stored
    pa[j] = g.A + (size_t)am * g.lda + c * 8 + (size_t)kchunk * kc;
  }
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int i = tid + THREADS * j;
    const int row = i >> 3, c = i & 7;
    slot_w[j] = lds_slot(row, c);
    int wr;
    if constexpr (EPI == EPI_SWIGLU) {
      // 32-row slices alternate gate / up for the same 32 outputs
      const int s = row >> 5;
      wr = tn * (BN / 2) + (s >> 1) * 32 + (row & 31) + (s & 1) * g.F;
    } else {
      wr = tn * BN + row;
    }
    pw[j] = g.W + (size_t)wr * g.ldw + c * 8 + (size_t)kchunk * kc;
  }

  f32x16 acc[FS][TS];
#pragma unroll
  for (int a = 0; a < FS; ++a)
#pragma unroll
    for (int b = 0; b < TS; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  // Two register stages in flight: the K slice used at step kt+2 is fetched
  // from global memory at step kt and written to LDS at the end of step kt+1,
  // so its latency is covered by two steps of MFMA work (the K loop is
  // unrolled by two to keep the stage registers static).
  u32x4 ra[2][CA], rw[2][CW];
  const int nk = kc / BK;

  auto gload = [&](int st, int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int j = 0; j < CA; ++j) ra[st][j] = *(const u32x4 *)(pa[j] + k0);
#pragma unroll
    for (int j = 0; j < CW; ++j) rw[st][j] = *(const u32x4 *)(pw[j] + k0);
  };
  auto lstore = [&](int st, int b) {
#pragma unroll
    for (int j = 0; j < CA; ++j) sA[b][slot_a[j]] = ra[st][j];
#pragma unroll
    for (int j = 0; j < CW; ++j) sW[b][slot_w[j]] = rw[st][j];
  };
  auto compute = [&](int b) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      u32x4 af[FS], bt[TS];
#pragma unroll
      for (int f = 0; f < FS; ++f) af[f] = sW[b][lds_slot(wn * WF + f * 32 + (lane & 31), ch)];
#pragma unroll
      for (int t = 0; t < TS; ++t) bt[t] = sA[b][lds_slot(wm * WT + t * 32 + (lane & 31), ch)];
#pragma unroll
      for (int f = 0; f < FS; ++f)
#pragma unroll
        for (int t = 0; t < TS; ++t) acc[f][t] = mfma32x32x16(af[f], bt[t], acc[f][t]);
    }
  };
  // step kt: stage kt sits in LDS buffer (kt & 1); register set (kt & 1) is
  // free, register set ((kt + 1) & 1) holds slice kt+1 in flight.
  auto step = [&](int kt, auto par) {
    constexpr int P = decltype(par)::value;
    if (kt + 2 < nk) gload(P, kt + 2);
    compute(P);
    if (kt + 1 < nk) lstore(P ^ 1, P ^ 1);
    __syncthreads();
  };

  gload(0, 0);
  if (nk > 1) gload(1, 1);
  lstore(0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>{});
  }

  // lane holds, for each (f, t) subtile and j = 0..3, the 4 consecutive
  // W rows f*32 + 8j + 4*(lane/32) + 0..3 of token t*32 + lane%32
  const int h4 = 4 * (lane >> 5);
  if constexpr (EPI == EPI_QKV) {
    static_assert(BM == 128 && BN == 128, "the epilogue's LDS objects are the two operand arrays");
    qkv_epilogue<BM, THREADS, TS, FS>(g, m0, tn * BN, wm * WT, tn * BN + wn * WF, acc, tid,
                                      LdsObjs<2>{&sA[0][0], &sW[0][0], nullptr, nullptr});
    return;
  }
#pragma unroll
  for (int t = 0; t < TS; ++t) {
    const int m = m0 + wm * WT + t * 32 + (lane & 31);
    if (m >= g.M) continue;
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int p = 0; p < FS / 2; ++p)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          store4_swiglu(g, m, tn * (BN / 2) + wn * (WF / 2) + p * 32 + 8 * j + h4, quad(acc[2 * p][t], j),
                        quad(acc[2 * p + 1][t], j));
    } else if (split) {
      float *prow = g.part + ((size_t)kchunk * g.M + m) * g.N;
#pragma unroll
      for (int f = 0; f < FS; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) *(f32x4 *)(prow + tn * BN + wn * WF + f * 32 + 8 * j + h4) = quad(acc[f][t], j);
    } else {
#pragma unroll
      for (int f = 0; f < FS; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) store4<EPI>(g, m, tn * BN + wn * WF + f * 32 + 8 * j + h4, quad(acc[f][t], j));
    }
  }
}

// The residual update of a K-split GEMM: x[m][n] += gate[row kind][n] *
// (((P_0 + P_1) + P_2) + ...)[m][n], the chunks summed in order in fp32.
// One thread per 4 consecutive outputs.
__global__ __launch_bounds__(256) void resid_reduce_kernel(const GemmArgs g) {
  if (g.skip && *g.skip) return;
  const int n4 = g.N >> 2;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)g.M * n4) return;
  const int m = (int)(i / n4), n = (int)(i % n4) * 4;
  const size_t mn = (size_t)g.M * g.N;
  const float *p = g.part + (size_t)m * g.N + n;
  f32x4 v = *(const f32x4 *)p;
  for (int s = 1; s < g.ksplit; ++s) v += *(const f32x4 *)(p + s * mn);
  const float *gp = g.gate + (m < g.L_rows ? 0 : g.gate_img_off) + n;
  f32x4 *xp = (f32x4 *)(g.X + (size_t)m * g.ldx + n);
  *xp = gated_add(*xp, *(const f32x4 *)gp, v);
}

// ---------------------------------------------------------------- 128 x 256 tiles, 8 waves
// A few hundred token rows: one 128 x 256 tile per workgroup of 8 waves (2
// along tokens x 4 along W rows; wave tile 64 tokens x 64 W rows, MFMA
// 32x32x16), one workgroup per CU -- 3/4 of the copied bytes per FLOP of two
// 128 x 128 workgroups.  (The 256 x 256 shape runs on gemm_bf16_lds_kernel
// below.)  On this shape the 32x32x16 MFMA runs faster than the 16x16x32 one
// of the 256 x 256 kernel, and both give the same fp32 results bit for bit.
//
// Operands go from global memory straight into LDS (buffer loads with the LDS
// flag: lane l of a copy instruction lands 16 bytes at slot base + l), so no
// register staging and no LDS store instructions: measured on gfx950, a
// ds_write_b128 costs the LDS about 2.5x a ds_read_b128 per byte, and with
// register staging the stores held the K loop to ~70% of MFMA rate.
// Each K step of 64 moves a BMT-row A slice and a 32 KB W slice.  The A
// slices (activations, just written by the previous kernel, mostly cache
// hits) are double-buffered and copied one step ahead; the W slices (weights,
// streamed from HBM) are triple-buffered and copied two steps ahead, so a W
// copy has two steps of MFMA work to land.  The five stages are separate LDS
// objects indexed by compile-time constants (the K loop is unrolled by 6), so
// the compiler's wait for a copy covers exactly the stage it fills, and the
// barrier that ends a step waits only for the copies that the next step
// reads, leaving the newest W copy in flight.
//
// LDS layout of a slice: row r (64 bf16 = 8 chunks of 16 bytes), chunk c at
// slot r * 8 + (c ^ ((r >> 1) & 7)) (see lds_slot).  Copy instruction j of
// wave w fills slots (8 j + w) * 64 .. + 63: rows 64 j + 8 w + lane / 8, slot
// lane % 8 holding chunk (lane % 8) ^ ((row >> 1) & 7) -- which does not
// depend on j -- so each lane's W source offset is fixed and j only adds a
// uniform 64-row step.  Token rows past M are clamped to row M - 1 (loaded,
// never stored), so every copy stays inside the operands.
//
// EPI_RESID may split K: as in the 128 x 128 kernels, chunk s of K writes
// fp32 partial sums and resid_reduce_kernel adds them in order.
namespace gemmL {
constexpr int BN = 256, BK = 64, THREADS = 512;
constexpr int FS = 2;                   // wave tile: 2 x 32 W rows
constexpr int NCP = BN * 8 / THREADS;   // W copy instructions per slice per thread (4)
constexpr int RSRC_FLAGS = 0x00020000;  // raw buffer, 32-bit dwords
}  // namespace gemmL

template <int EPI, int WMN, int WNN, int BMT = 128>
__global__ __launch_bounds__(gemmL::THREADS, 1) void gemm_bf16_large_kernel(const GemmArgs g) {
  using namespace gemmL;
  static_assert(WMN == 2 && WNN == 4, "8 waves as 2 x 4");
  static_assert(BMT == 128, "128 token rows (256-row tiles run on gemm_bf16_lds_kernel)");
  if (g.skip && *g.skip) return;
  constexpr int BM = BMT, TS = BM / (WMN * 32);
  constexpr int NCPA = BM * 8 / THREADS;  // A copy instructions per slice per thread (4 or 2)
  constexpr int WT = BM / WMN, WF = BN / WNN;
  __shared__ u32x4 sA0[BM * 8], sA1[BM * 8];
  __shared__ u32x4 sW0[BN * 8], sW1[BN * 8], sW2[BN * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WMN, wn = wave / WMN;
  const int nTM = (g.M + BM - 1) / BM;
  const int nTN = EPI == EPI_SWIGLU ? g.F / (BN / 2) : g.N / BN;
  const bool split = EPI == EPI_RESID && g.ksplit > 1;
  const int ntile = nTM * nTN;
  const int kchunk = split ? (int)(blockIdx.x / ntile) : 0;
  const int kc = split ? g.K / g.ksplit : g.K;
  int tm, tn;
  tile_of(split ? (int)(blockIdx.x % ntile) : (int)blockIdx.x, nTM, nTN, tm, tn);
  const int m0 = tm * BM;

  // copy sources: tile row r0 + 64 j, chunk cch
  const int r0 = 8 * wave + (lane >> 3);
  const int cch = (lane & 7) ^ ((r0 >> 1) & 7);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void *)g.A, (short)0, (int)((size_t)g.M * g.lda * 2), RSRC_FLAGS);
  const int wrows = EPI == EPI_SWIGLU ? 2 * g.F : g.N;
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void *)g.W, (short)0, (int)((size_t)wrows * g.ldw * 2), RSRC_FLAGS);
  int voff_a[NCPA];
#pragma unroll
  for (int j = 0; j < NCPA; ++j) voff_a[j] = (min(m0 + r0 + 64 * j, g.M - 1) * g.lda + cch * 8) * 2;
  // SwiGLU: W tile rows alternate 32-row gate / up slices for the same 32
  // outputs: tile row r reads W row tn*128 + (r>>6)*32 + (r&31) (+F when bit
  // 5 of r is set); for r = r0 + 64 j that is a per-lane part plus 32 j.
  const int wrow0 = EPI == EPI_SWIGLU ? tn * (BN / 2) + (r0 & 31) + ((r0 >> 5) & 1) * g.F : tn * BN + r0;
  const int voff_w = (wrow0 * g.ldw + cch * 8) * 2;
  const int wstep = (EPI == EPI_SWIGLU ? 32 : 64) * g.ldw * 2;  // bytes per copy instruction j
  const int kbase = kchunk * kc * 2;                            // the chunk's first K column, bytes
  auto lds_ptr = [](u32x4 *p) { return (__attribute__((address_space(3))) void *)p; };
  auto copy_a = [&](int kt, u32x4 *dst) {
#if __HIP_DEVICE_COMPILE__  // the host pass cannot resolve this builtin in a template
#pragma unroll
    for (int j = 0; j < NCPA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds_ptr(dst + (8 * j + wave) * 64), 16, voff_a[j],
                                               kbase + kt * BK * 2, 0, 0);
#endif
  };
  auto copy_w = [&](int kt, u32x4 *dst) {
#if __HIP_DEVICE_COMPILE__
#pragma unroll
    for (int j = 0; j < NCP; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, lds_ptr(dst + (8 * j + wave) * 64), 16, voff_w,
                                               wstep * j + kbase + kt * BK * 2, 0, 0);
#endif
  };

  f32x16 acc[FS][TS];
#pragma unroll
  for (int a = 0; a < FS; ++a)
#pragma unroll
    for (int b = 0; b < TS; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  // fragment rows: (wave base + 32 i + lane % 32); swizzle term depends on lane only
  const int fr = lane & 31, sw = (fr >> 1) & 7, half = lane >> 5;
  const int rowA = wm * WT + fr, rowW = wn * WF + fr;
  u32x4 fa[2][TS], fw[2][FS];
  auto fload = [&](const u32x4 *sa, const u32x4 *sw_, int kk, int set) {
    const int ch = (kk * 2 + half) ^ sw;
#pragma unroll
    for (int t = 0; t < TS; ++t) fa[set][t] = sa[(rowA + 32 * t) * 8 + ch];
#pragma unroll
    for (int f = 0; f < FS; ++f) fw[set][f] = sw_[(rowW + 32 * f) * 8 + ch];
  };
  auto mfma_kk = [&](int set) {
#pragma unroll
    for (int f = 0; f < FS; ++f)
#pragma unroll
      for (int t = 0; t < TS; ++t) acc[f][t] = mfma32x32x16(fw[set][f], fa[set][t], acc[f][t]);
  };
  // n MFMAs, each followed by up to one LDS read and one copy issued next to
  // it in program order
  auto interleave = [&](auto n_mfma, auto n_rd, auto n_cp) {
    constexpr int NM = decltype(n_mfma)::value, NR = decltype(n_rd)::value, NC = decltype(n_cp)::value;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // one MFMA
      if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      if (i < NC) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one copy
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using IM = std::integral_constant<int, FS * TS>;
  using IR = std::integral_constant<int, FS + TS>;
  using IC = std::integral_constant<int, NCP>;
  // stage objects by compile-time index
  auto SA = [&](auto i) -> u32x4 * {
    if constexpr (decltype(i)::value == 0) return sA0;
    else return sA1;
  };
  auto SW = [&](auto i) -> u32x4 * {
    if constexpr (decltype(i)::value == 0) return sW0;
    else if constexpr (decltype(i)::value == 1) return sW1;
    else return sW2;
  };
  using std::integral_constant;

  const int nk = kc / BK;
  // Step kt reads A stage PA = kt % 2 and W stage PW = kt % 3 (sub-step 0's
  // fragments already in register set 0).  It first copies A slice kt+1 into
  // the other A stage, then (strictly after, in issue order) W slice kt+2
  // into W stage (kt+2) % 3 -- both stages read by step kt-1 and released by
  // its barrier; past the last slice the copies repeat slice nk-1 into a
  // stage never read again.  The step ends with every copy but the NCP
  // newest (W slice kt+2) landed -- vector-memory loads complete in issue
  // order, so vmcnt(NCP) covers A slice kt+1 and W slice kt+1 -- and its own
  // LDS reads done, then the barrier, then the next step's sub-step 0
  // fragments.
  auto step = [&](int kt, auto pa, auto pw) {
    constexpr int PA = decltype(pa)::value, PW = decltype(pw)::value;
    const u32x4 *a = SA(pa), *w = SW(pw);
    copy_a(min(kt + 1, nk - 1), SA(integral_constant<int, PA ^ 1>{}));
    __builtin_amdgcn_sched_barrier(0);  // the A copies are issued before the W copies
    copy_w(min(kt + 2, nk - 1), SW(integral_constant<int, (PW + 2) % 3>{}));
    fload(a, w, 1, 1);
    mfma_kk(0);
    interleave(IM{}, IR{}, IC{});
    fload(a, w, 2, 0);
    mfma_kk(1);
    interleave(IM{}, IR{}, I0{});
    fload(a, w, 3, 1);
    mfma_kk(0);
    interleave(IM{}, IR{}, I0{});
    mfma_kk(1);
    // s_waitcnt vmcnt(NCP) expcnt(7) lgkmcnt(0), then the barrier
    __builtin_amdgcn_s_waitcnt((NCP & 15) | (7 << 4) | ((NCP >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    fload(SA(integral_constant<int, PA ^ 1>{}), SW(integral_constant<int, (PW + 1) % 3>{}), 0, 0);
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  copy_a(0, sA0);
  copy_w(0, sW0);
  __builtin_amdgcn_sched_barrier(0);  // slice 0 is issued before W slice 1
  copy_w(min(1, nk - 1), sW1);
  __builtin_amdgcn_s_waitcnt((NCP & 15) | (7 << 4) | ((NCP >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  fload(sA0, sW0, 0, 0);
  int kt = 0;
  for (; kt + 6 <= nk; kt += 6) {
    step(kt, C0{}, C0{});
    step(kt + 1, C1{}, C1{});
    step(kt + 2, C0{}, C2{});
    step(kt + 3, C1{}, C0{});
    step(kt + 4, C0{}, C1{});
    step(kt + 5, C1{}, C2{});
  }
  if (kt < nk) step(kt, C0{}, C0{});
  if (kt + 1 < nk) step(kt + 1, C1{}, C1{});
  if (kt + 2 < nk) step(kt + 2, C0{}, C2{});
  if (kt + 3 < nk) step(kt + 3, C1{}, C0{});
  if (kt + 4 < nk) step(kt + 4, C0{}, C1{});
  // every copy has landed (vmcnt(0) expcnt(7) lgkmcnt(0)) and every fragment
  // read is done before the epilogue reuses the stages
  __builtin_amdgcn_s_waitcnt(7 << 4);
  __syncthreads();

  const int h4 = 4 * half;
  if constexpr (EPI == EPI_QKV) {
    qkv_epilogue<BM, THREADS, TS, FS>(g, m0, tn * BN, wm * WT, tn * BN + wn * WF, acc, tid,
                                      LdsObjs<4, BM * 8>{sA0, sA1, sW0, sW1});
    return;
  }
#pragma unroll
  for (int t = 0; t < TS; ++t) {
    const int m = m0 + wm * WT + t * 32 + fr;
    if (m >= g.M) continue;
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int p = 0; p < FS / 2; ++p)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          store4_swiglu(g, m, tn * (BN / 2) + wn * (WF / 2) + p * 32 + 8 * j + h4, quad(acc[2 * p][t], j),
                        quad(acc[2 * p + 1][t], j));
    } else if (split) {
      float *prow = g.part + ((size_t)kchunk * g.M + m) * g.N;
#pragma unroll
      for (int f = 0; f < FS; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) *(f32x4 *)(prow + tn * BN + wn * WF + f * 32 + 8 * j + h4) = quad(acc[f][t], j);
    } else {
#pragma unroll
      for (int f = 0; f < FS; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) store4<EPI>(g, m, tn * BN + wn * WF + f * 32 + 8 * j + h4, quad(acc[f][t], j));
    }
  }
}

// ---------------------------------------------------------------- 128 x 128 tiles, LDS copies
// Small-M shape with the large kernel's operand path.  A few hundred token
// rows give too few 256 x 256 tiles for 256 CUs, so the tile stays 128 x 128
// (4 waves as 2 x 2, wave tile 64 tokens x 64 W rows, two workgroups per CU):
// exactly the MFMA sequence of gemm_bf16_kernel<EPI, 128, 128>, hence the
// same bits.  What changes is how the operands reach LDS.  With register
// staging each K step writes its 32 KB of slices with ds_write, which the
// LDS serves at about 2.5x the cost of a read per byte; together with one
// fragment read per MFMA (a 64 x 64 wave tile reads 4 fragments for 4
// MFMAs) that held the small kernel to about 45% of the MFMA rate.  Here the
// slices are copied global -> LDS directly, A double-buffered one step ahead
// and W triple-buffered two steps ahead, five 16 KB LDS objects (80 KB per
// workgroup, two workgroups fill the 160 KB), with the large kernel's copy
// order and waits.  Copy instruction j of wave w fills slots (4 j + w) * 64
// .. + 63: tile rows 32 j + 8 w + lane / 8, chunk (lane % 8) ^ ((row >> 1) & 7)
// -- independent of j.  Token rows past M are clamped to row M - 1 (loaded,
// never stored), so every copy stays inside the operands.
namespace gemmM {
constexpr int BM = 128, BN = 128, BK = 64, THREADS = 256;
constexpr int TS = 2, FS = 2;           // wave tile: 2 x 32 tokens, 2 x 32 W rows
constexpr int NCP = BM * 8 / THREADS;   // copy instructions per operand slice per thread (4)
constexpr int RSRC_FLAGS = 0x00020000;  // raw buffer, 32-bit dwords
}  // namespace gemmM

template <int EPI>
__global__ __launch_bounds__(gemmM::THREADS, 2) void gemm_bf16_mid_kernel(const GemmArgs g) {
  using namespace gemmM;
  if (g.skip && *g.skip) return;
  constexpr int WT = BM / 2, WF = BN / 2;
  __shared__ u32x4 sA0[BM * 8], sA1[BM * 8];
  __shared__ u32x4 sW0[BN * 8], sW1[BN * 8], sW2[BN * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int nTM = (g.M + BM - 1) / BM;
  const int nTN = EPI == EPI_SWIGLU ? g.F / (BN / 2) : g.N / BN;
  // split over K (EPI_RESID only): the workgroup's chunk and its K columns
  const bool split = EPI == EPI_RESID && g.ksplit > 1;
  const int ntile = nTM * nTN;
  const int kchunk = split ? (int)(blockIdx.x / ntile) : 0;
  const int kc = split ? g.K / g.ksplit : g.K;
  int tm, tn;
  tile_of(split ? (int)(blockIdx.x % ntile) : (int)blockIdx.x, nTM, nTN, tm, tn);
  const int m0 = tm * BM;

  // copy sources: tile row r0 + 32 j, chunk cch
  const int r0 = 8 * wave + (lane >> 3);
  const int cch = (lane & 7) ^ ((r0 >> 1) & 7);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void *)g.A, (short)0, (int)((size_t)g.M * g.lda * 2), RSRC_FLAGS);
  const int wrows = EPI == EPI_SWIGLU ? 2 * g.F : g.N;
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void *)g.W, (short)0, (int)((size_t)wrows * g.ldw * 2), RSRC_FLAGS);
  int voff_a[NCP];
#pragma unroll
  for (int j = 0; j < NCP; ++j) voff_a[j] = (min(m0 + r0 + 32 * j, g.M - 1) * g.lda + cch * 8) * 2;
  // SwiGLU: 32-row W slices alternate gate / up for the same 32 outputs; tile
  // row 32 j + r0 (r0 < 32) reads W row tn*64 + (j>>1)*32 + r0 (+F for odd j)
  const int wrow0 = EPI == EPI_SWIGLU ? tn * (BN / 2) + r0 : tn * BN + r0;
  const int voff_w = (wrow0 * g.ldw + cch * 8) * 2;
  auto wrow_step = [&](int j) {
    return EPI == EPI_SWIGLU ? ((j >> 1) * 32 + (j & 1) * g.F) * g.ldw * 2 : 32 * j * g.ldw * 2;
  };
  const int kbase = kchunk * kc * 2;  // byte offset of the chunk's first K column
  auto lds_ptr = [](u32x4 *p) { return (__attribute__((address_space(3))) void *)p; };
  auto copy_a = [&](int kt, u32x4 *dst) {
#if __HIP_DEVICE_COMPILE__  // the host pass cannot resolve this builtin in a template
#pragma unroll
    for (int j = 0; j < NCP; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds_ptr(dst + (4 * j + wave) * 64), 16, voff_a[j],
                                               kbase + kt * BK * 2, 0, 0);
#endif
  };
  auto copy_w = [&](int kt, u32x4 *dst) {
#if __HIP_DEVICE_COMPILE__
#pragma unroll
    for (int j = 0; j < NCP; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, lds_ptr(dst + (4 * j + wave) * 64), 16, voff_w,
                                               wrow_step(j) + kbase + kt * BK * 2, 0, 0);
#endif
  };

  f32x16 acc[FS][TS];
#pragma unroll
  for (int a = 0; a < FS; ++a)
#pragma unroll
    for (int b = 0; b < TS; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  const int fr = lane & 31, sw = (fr >> 1) & 7, half = lane >> 5;
  const int rowA = wm * WT + fr, rowW = wn * WF + fr;
  u32x4 fa[2][TS], fw[2][FS];
  auto fload = [&](const u32x4 *sa, const u32x4 *sw_, int kk, int set) {
    const int ch = (kk * 2 + half) ^ sw;
#pragma unroll
    for (int f = 0; f < FS; ++f) fw[set][f] = sw_[(rowW + 32 * f) * 8 + ch];
#pragma unroll
    for (int t = 0; t < TS; ++t) fa[set][t] = sa[(rowA + 32 * t) * 8 + ch];
  };
  auto mfma_kk = [&](int set) {
#pragma unroll
    for (int f = 0; f < FS; ++f)
#pragma unroll
      for (int t = 0; t < TS; ++t) acc[f][t] = mfma32x32x16(fw[set][f], fa[set][t], acc[f][t]);
  };
  auto interleave = [&](auto n_mfma, auto n_rd, auto n_cp) {
    constexpr int NM = decltype(n_mfma)::value, NR = decltype(n_rd)::value, NC = decltype(n_cp)::value;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // one MFMA
      if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      if (i < NC) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one copy
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I4 = std::integral_constant<int, FS * TS>;
  using IR = std::integral_constant<int, FS + TS>;
  using IC = std::integral_constant<int, NCP>;
  auto SA = [&](auto i) -> u32x4 * {
    if constexpr (decltype(i)::value == 0) return sA0;
    else return sA1;
  };
  auto SW = [&](auto i) -> u32x4 * {
    if constexpr (decltype(i)::value == 0) return sW0;
    else if constexpr (decltype(i)::value == 1) return sW1;
    else return sW2;
  };
  using std::integral_constant;

  const int nk = kc / BK;
  // Step kt: the large kernel's step (A slice kt+1 and W slice kt+2 copied
  // into the stages step kt-1 released, the barrier waits for all but the
  // newest W copy).
  auto step = [&](int kt, auto pa, auto pw) {
    constexpr int PA = decltype(pa)::value, PW = decltype(pw)::value;
    const u32x4 *a = SA(pa), *w = SW(pw);
    copy_a(min(kt + 1, nk - 1), SA(integral_constant<int, PA ^ 1>{}));
    __builtin_amdgcn_sched_barrier(0);  // the A copies are issued before the W copies
    copy_w(min(kt + 2, nk - 1), SW(integral_constant<int, (PW + 2) % 3>{}));
    fload(a, w, 1, 1);
    mfma_kk(0);
    interleave(I4{}, IR{}, IC{});
    fload(a, w, 2, 0);
    mfma_kk(1);
    interleave(I4{}, IR{}, I0{});
    fload(a, w, 3, 1);
    mfma_kk(0);
    interleave(I4{}, IR{}, I0{});
    mfma_kk(1);
    // s_waitcnt vmcnt(NCP) expcnt(7) lgkmcnt(0), then the barrier
    __builtin_amdgcn_s_waitcnt((NCP & 15) | (7 << 4) | ((NCP >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    fload(SA(integral_constant<int, PA ^ 1>{}), SW(integral_constant<int, (PW + 1) % 3>{}), 0, 0);
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  copy_a(0, sA0);
  copy_w(0, sW0);
  __builtin_amdgcn_sched_barrier(0);  // slice 0 is issued before W slice 1
  copy_w(min(1, nk - 1), sW1);
  __builtin_amdgcn_s_waitcnt((NCP & 15) | (7 << 4) | ((NCP >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  fload(sA0, sW0, 0, 0);
  int kt = 0;
  for (; kt + 6 <= nk; kt += 6) {
    step(kt, C0{}, C0{});
    step(kt + 1, C1{}, C1{});
    step(kt + 2, C0{}, C2{});
    step(kt + 3, C1{}, C0{});
    step(kt + 4, C0{}, C1{});
    step(kt + 5, C1{}, C2{});
  }
  if (kt < nk) step(kt, C0{}, C0{});
  if (kt + 1 < nk) step(kt + 1, C1{}, C1{});
  if (kt + 2 < nk) step(kt + 2, C0{}, C2{});
  if (kt + 3 < nk) step(kt + 3, C1{}, C0{});
  if (kt + 4 < nk) step(kt + 4, C0{}, C1{});
  // every copy has landed (vmcnt(0) expcnt(7) lgkmcnt(0)) and every fragment
  // read is done before the epilogue reuses the stages
  __builtin_amdgcn_s_waitcnt(7 << 4);
  __syncthreads();

  const int h4 = 4 * half;
  if constexpr (EPI == EPI_QKV) {
    qkv_epilogue<BM, THREADS, TS, FS>(g, m0, tn * BN, wm * WT, tn * BN + wn * WF, acc, tid,
                                      LdsObjs<4, BM * 8>{sA0, sA1, sW0, sW1});
    return;
  }
#pragma unroll
  for (int t = 0; t < TS; ++t) {
    const int m = m0 + wm * WT + t * 32 + fr;
    if (m >= g.M) continue;
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int p = 0; p < FS / 2; ++p)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          store4_swiglu(g, m, tn * (BN / 2) + wn * (WF / 2) + p * 32 + 8 * j + h4, quad(acc[2 * p][t], j),
                        quad(acc[2 * p + 1][t], j));
    } else if (split) {
      float *prow = g.part + ((size_t)kchunk * g.M + m) * g.N;
#pragma unroll
      for (int f = 0; f < FS; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) *(f32x4 *)(prow + tn * BN + wn * WF + f * 32 + 8 * j + h4) = quad(acc[f][t], j);
    } else {
#pragma unroll
      for (int f = 0; f < FS; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) store4<EPI>(g, m, tn * BN + wn * WF + f * 32 + 8 * j + h4, quad(acc[f][t], j));
    }
  }
}

// ---------------------------------------------------------------- 256 x 256 tiles, 16x16x32 MFMA
// Large M: one 256 x 256 tile per workgroup of 8 waves (2 along tokens x 4
// along W rows, wave tile 128 tokens x 64 W rows -- half a q / k / v head,
// one gate and one up half of 32 SwiGLU outputs), one workgroup per CU.
//
// MFMA 16x16x32 bf16, issued as D[16 W rows][16 tokens]: lane l holds the 4
// consecutive W rows 4 (l / 16) .. + 3 of token l % 16, so RoPE pairs and
// float4 residual updates stay inside a lane, and one store instruction
// covers 16 tokens x 16 consecutive features.  Against the 32x32x16 shape of
// the other kernels it takes half the K per instruction and the same LDS
// reads per FLOP; on the MI355X both shapes give the same fp32 result bit for
// bit (checked over random and rounding-sensitive inputs, and on whole DiT
// steps against the register-staged kernel), and on this tile the 16x16x32
// form runs the gate/up, QKV and O-proj GEMMs 5-7% faster.
//
// Operands go from global memory straight into LDS (buffer loads with the LDS
// flag: lane l of a copy instruction lands 16 bytes at slot base + l), so no
// register staging and no LDS store instructions: measured on gfx950, a
// ds_write_b128 costs the LDS about 2.5x a ds_read_b128 per byte.  Each K step
// of 64 moves a 256-row A slice and a 256-row W slice.  The A slices
// (activations, just written by the previous kernel, mostly cache hits) are
// double-buffered, the W slices (weights, streamed from HBM) triple-buffered;
// step k copies W slice k+2 during its first half and A slice k+2 during its
// second, one copy instruction per few MFMAs.  The five stages are separate
// LDS objects indexed by compile-time constants (the K loop is unrolled by
// 6).  Each step has one barrier, in its middle, once its stages are read
// (see the K loop).
//
// LDS layout of a slice: row r (64 bf16 = 8 chunks of 16 bytes), chunk c at
// slot r * 8 + (c ^ ((r >> 1) & 7)) (see lds_slot).  Copy instruction j of
// wave w fills slots (8 j + w) * 64 .. + 63: rows 64 j + 8 w + lane / 8,
// slot lane % 8 holding chunk (lane % 8) ^ ((row >> 1) & 7) -- which does not
// depend on j -- so each lane's source offset is fixed and j only adds a
// uniform 64-row step.  Token rows past M are clamped to row M - 1
// (loaded, never stored), so every copy stays inside the operands.  A
// fragment (16 rows x 32 K) is one ds_read_b128 per lane: row l % 16, chunk
// 4 kk + l / 16 of sub-step kk; the 16 rows of one read pass land on 16
// distinct 16-byte bank groups.
//
// EPI_RESID may split K: chunk s of K writes fp32 partial sums and
// resid_reduce_kernel adds them in order.
namespace gemmT {
constexpr int BK = 64;
constexpr int RSRC_FLAGS = 0x00020000;  // raw buffer, 32-bit dwords
}  // namespace gemmT

// MFMAs per interleaved instruction when n of them go among nm MFMAs
constexpr int spacing(int nm, int n) { return n > 0 && nm / n > 0 ? nm / n : 1; }

template <int N, int I = 0, class F>
QI_DEV void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// The V section of a QKV wave tile: NW = 4 blocks of 16 W rows from n0 (one
// head, n0 % 64 == 0) and NT blocks of 16 tokens from mbase, stored
// transposed into V^T [heads][128][ldv]: for one output feature the 16 lanes
// l % 16 hold 16 consecutive tokens (32 contiguous bytes per store).
template <int NT, int NW>
QI_DEV void store_v_wave16(const GemmArgs &g, int mbase, int n0, const f32x4 (&acc)[NW][NT], int lane) {
  const int w0 = n0 - 2 * g.H;
  const int head = w0 >> 7, dh0 = w0 & 127;
  const int fr = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int m = mbase + 16 * t + fr;
    if (m >= g.M) continue;
    const bool txt = m < g.L_rows;
    const int row = txt ? m : m - g.L_rows;
    const int br = (txt || g.batch <= 1) ? 0 : row / g.seg_i;  // branch of an image row
    const int brow = row - br * g.seg_i;
    const int ldv = txt ? g.ldv_t : g.ldv_i;
    u16 *base =
        (txt ? g.vt_t : g.vt_i) + (size_t)br * g.H * ldv + ((size_t)head * 128 + dh0 + 4 * kq) * ldv + brow;
#pragma unroll
    for (int f = 0; f < NW; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) base[(size_t)(16 * f + r) * ldv] = f32_to_bf16(acc[f][t][r]);
  }
}

// The QKV epilogue of a BM-token workgroup tile of the 256 x 256 kernel (the
// qkv_epilogue steps with the 16x16 accumulator layout): wave (wrow / WT,
// n0) holds WT = 16 NT tokens x 64 W rows, half of one q or k head, as 4
// consecutive features of one token per lane and accumulator.  The caller
// has loaded the tile's RoPE rows (q / k tiles) and passed a barrier after
// which the LDS is free.
template <int BM, int THREADS, int NT, int NW, int NOBJ, int SLOTS>
QI_DEV void qkv_epilogue16(const GemmArgs &g, int m0, int n_tile, int wrow, int n0, const f32x4 (&acc)[NW][NT],
                           int tid, const LdsObjs<NOBJ, SLOTS> lo, const RopeRows<BM, THREADS> &rope) {
  static_assert(NW == 4, "a wave tile is half a head: 64 W rows");
  constexpr int R = LdsObjs<NOBJ, SLOTS>::kRows;
  constexpr int WT = 16 * NT;
  constexpr int RS = WT * 8;       // 16-byte slots of one wave's region
  constexpr int RPO = SLOTS / RS;  // regions per object
  static_assert(RPO >= 1 && (THREADS / 64) <= RPO * NOBJ, "the waves' regions fit in the objects");
  const int lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, kq = lane >> 4;
  if (n_tile / g.H >= 2) {
    store_v_wave16<NT, NW>(g, m0 + wrow, n0, acc, lane);
    return;
  }
  const int sec = n0 / g.H;
  const int w0 = n0 - sec * g.H;
  const int head = w0 >> 7, dh0 = w0 & 127;
  rope.store(g, m0, lo, tid);  // the caller's barrier freed the LDS
  __syncthreads();
  // outputs dh0 + 16 f + 4 kq + 0..3 are RoPE pairs 2q, 2q + 1 with
  // q = dh0 / 4 + 4 f + kq
  const int q0 = (dh0 >> 2) + kq;
  u32x2 y[NT][NW];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = wrow + 16 * t + fr;
    const u32x2 *cl2 = (const u32x2 *)lo.o(r / R), *sl2 = (const u32x2 *)lo.o(BM / R + r / R);
#pragma unroll
    for (int f = 0; f < NW; ++f) {
      const int slot = (r % R) * 32 + ((q0 + 4 * f) ^ (r & 31));
      const float2 cs = __builtin_bit_cast(float2, cl2[slot]);
      const float2 sn = __builtin_bit_cast(float2, sl2[slot]);
      const f32x4 v = acc[f][t];
      const float2 y01 = rope_pair(v[0], v[1], cs.x, sn.x), y23 = rope_pair(v[2], v[3], cs.y, sn.y);
      y[t][f] = u32x2{pack_bf16x2(y01.x, y01.y), pack_bf16x2(y23.x, y23.y)};
    }
  }
  __syncthreads();  // every wave is done with the staged tables
  u32x4 *reg = lo.o(wave / RPO) + (wave % RPO) * RS;
  u32x2 *reg2 = (u32x2 *)reg;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int rr = 16 * t + fr;
#pragma unroll
    for (int f = 0; f < NW; ++f) reg2[rr * 16 + ((4 * f + kq) ^ ((rr >> 1) & 15))] = y[t][f];
  }
  __syncthreads();
  u16 *qk_t = sec == 0 ? g.q_t : g.k_t, *qk_i = sec == 0 ? g.q_i : g.k_i;
#pragma unroll
  for (int it = 0; it < WT * 8 / 64; ++it) {
    const int i = lane + 64 * it;
    const int rr = i >> 3, k = i & 7, x = (rr >> 1) & 15;
    u32x4 v = reg[rr * 8 + (k ^ (x >> 1))];
    if (x & 1) v = u32x4{v[2], v[3], v[0], v[1]};
    const int m = m0 + wrow + rr;
    if (m >= g.M) continue;
    const bool txt = m < g.L_rows;
    const int row = txt ? m : m - g.L_rows;
    const int br = (txt || g.batch <= 1) ? 0 : row / g.seg_i;  // branch of an image row
    const int brow = row - br * g.seg_i;
    u16 *dst = (txt ? qk_t : qk_i) + (size_t)br * g.H * g.seg_i +
               ((size_t)head * (txt ? g.seg_t : g.seg_i) + brow) * 128 + dh0 + 8 * k;
    *(u32x4 *)dst = v;
  }
}

template <int EPI, int BM, int BN, int WAVES>
__global__ __launch_bounds__(64 * WAVES, WAVES == 8 ? 1 : 2) void gemm_bf16_lds_kernel(const GemmArgs g) {
  using namespace gemmT;
  static_assert(BM == 256 && BN == 256 && WAVES == 8, "the 256 x 256 tile");
  constexpr int THREADS = 64 * WAVES, WN = WAVES / 2;
  constexpr int WT = BM / 2, WF = BN / WN;  // wave tile: WT tokens x WF W rows
  constexpr int NT = WT / 16, NW = WF / 16;
  static_assert(WF == 64, "a wave tile holds 64 W rows");
  constexpr int NCPA = BM * 8 / THREADS, NCPW = BN * 8 / THREADS;  // copy instructions per slice per thread
  constexpr int RSTEP = 8 * WAVES;                                 // tile rows per copy instruction
  if (g.skip && *g.skip) return;
  __shared__ u32x4 sA0[BM * 8], sA1[BM * 8];
  __shared__ u32x4 sW0[BN * 8], sW1[BN * 8], sW2[BN * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int nTM = (g.M + BM - 1) / BM;
  const int nTN = EPI == EPI_SWIGLU ? g.F / (BN / 2) : g.N / BN;
  const bool split = EPI == EPI_RESID && g.ksplit > 1;
  const int ntile = nTM * nTN;
  const int kchunk = split ? (int)(blockIdx.x / ntile) : 0;
  const int kc = split ? g.K / g.ksplit : g.K;
  int tm, tn;
  tile_of(split ? (int)(blockIdx.x % ntile) : (int)blockIdx.x, nTM, nTN, tm, tn);
  const int m0 = tm * BM;

  // copy sources: tile row r0 + RSTEP j, chunk cch
  const int r0 = 8 * wave + (lane >> 3);
  const int cch = (lane & 7) ^ ((r0 >> 1) & 7);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void *)g.A, (short)0, (int)((size_t)g.M * g.lda * 2), RSRC_FLAGS);
  const int wrows = EPI == EPI_SWIGLU ? 2 * g.F : g.N;
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void *)g.W, (short)0, (int)((size_t)wrows * g.ldw * 2), RSRC_FLAGS);
  int voff_a[NCPA];
#pragma unroll
  for (int j = 0; j < NCPA; ++j) voff_a[j] = (min(m0 + r0 + RSTEP * j, g.M - 1) * g.lda + cch * 8) * 2;
  // SwiGLU: the tile's W rows alternate 32-row gate / up slices for the same
  // 32 outputs: tile row r reads W row tn * BN/2 + (r >> 6) * 32 + (r & 31),
  // plus F when bit 5 of r is set; for r = r0 + RSTEP j that is a per-lane
  // part plus a uniform step
  const int wrow0 = EPI == EPI_SWIGLU ? tn * (BN / 2) + (r0 & 31) + (RSTEP == 64 ? ((r0 >> 5) & 1) * g.F : 0)
                                      : tn * BN + r0;
  const int voff_w = (wrow0 * g.ldw + cch * 8) * 2;
  auto wstep = [&](int j) {  // bytes
    const int rows = EPI == EPI_SWIGLU ? (RSTEP == 64 ? 32 * j : (j >> 1) * 32 + (j & 1) * g.F) : RSTEP * j;
    return rows * g.ldw * 2;
  };
  const int kbase = kchunk * kc * 2;  // the chunk's first K column, bytes
  // LDS DMA issued through inline asm (M0 = the wave's LDS destination, then
  // buffer_load_dwordx4 ... lds).  The compiler then does not count these
  // copies as pending LDS writes: with the builtin it adds waits of its own
  // before fragment reads of other stages (down to vmcnt(0) where the
  // six-step groups join), which stall the pipeline.  The order is kept by
  // the explicit waits and barriers below: every stage is read only after the
  // wait and barrier that follow its copies, and copied into only after the
  // barrier that follows its last reads; nothing else in this kernel uses M0.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto dma = [&](const __amdgpu_buffer_rsrc_t &rs, u32x4 *dst, int voff, int soff) {
    const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)dst;
// clang warns that M0 is a reserved register; declaring it clobbered is what
// keeps the compiler from assuming its value across the statement
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(rs),
                 "s"(soff)
                 : "m0");
#pragma clang diagnostic pop
  };
  auto copy_a1 = [&](int kt, u32x4 *dst, int j) { dma(ra, dst + (WAVES * j + wv) * 64, voff_a[j], kbase + kt * BK * 2); };
  auto copy_w1 = [&](int kt, u32x4 *dst, int j) {
    dma(rw, dst + (WAVES * j + wv) * 64, voff_w, wstep(j) + kbase + kt * BK * 2);
  };

  f32x4 acc[NW][NT];
#pragma unroll
  for (int a = 0; a < NW; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment rows: wave base + 16 i + lane % 16; rows 16 i apart share the
  // swizzle term, so fragment i of sub-step kk sits at slot off[kk] + 128 i
  const int fr = lane & 15, kq = lane >> 4, sw = (fr >> 1) & 7;
  const int rowA = wm * WT + fr, rowW = wn * WF + fr;
  int offA[2], offW[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    offA[kk] = rowA * 8 + ((4 * kk + kq) ^ sw);
    offW[kk] = rowW * 8 + ((4 * kk + kq) ^ sw);
  }
  u32x4 fa[2][NT], fw[2][NW];
  auto fload = [&](const u32x4 *sa, const u32x4 *sw_, int kk, int set) {
#pragma unroll
    for (int t = 0; t < NT; ++t) fa[set][t] = sa[offA[kk] + 128 * t];
#pragma unroll
    for (int f = 0; f < NW; ++f) fw[set][f] = sw_[offW[kk] + 128 * f];
  };
  using std::integral_constant;
  auto SA = [&](auto i) -> u32x4 * {
    if constexpr (decltype(i)::value == 0) return sA0;
    else return sA1;
  };
  auto SW = [&](auto i) -> u32x4 * {
    if constexpr (decltype(i)::value == 0) return sW0;
    else if constexpr (decltype(i)::value == 1) return sW1;
    else return sW2;
  };
  // One sub-step's MFMAs (register set SET) in NC chunks: chunk c issues
  // copy instruction c, then runs its share of the MFMAs with its share of
  // the other sub-step's fragment reads (sub-step kk of stages ra_, rw_, into
  // the other register set) among them.  The scheduling barriers around each
  // chunk keep the copies one per NM / NC MFMAs: issued in a burst, the
  // copies held each wave's next MFMAs back behind them.
  auto phase = [&](auto set_c, const u32x4 *ra_, const u32x4 *rw_, int kk, auto nc, auto &&copy) {
    constexpr int SET = decltype(set_c)::value, NC = decltype(nc)::value;
    constexpr int NM = NW * NT, NR = NT + NW;
    static_for<NC>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      constexpr int m0 = c * NM / NC, m1 = (c + 1) * NM / NC, r0 = c * NR / NC, r1 = (c + 1) * NR / NC;
      copy(c);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = r0; r < r1; ++r) {
        if (r < NT) fa[1 - SET][r] = ra_[offA[kk] + 128 * r];
        else fw[1 - SET][r - NT] = rw_[offW[kk] + 128 * (r - NT)];
      }
#pragma unroll
      for (int m = m0; m < m1; ++m)
        acc[m / NT][m % NT] = mfma16x16x32(fw[SET][m / NT], fa[SET][m % NT], acc[m / NT][m % NT]);
      constexpr int CM = m1 - m0, CR = r1 - r0, RSP = spacing(CM, CR);
#pragma unroll
      for (int i = 0; i < CM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                    // one MFMA
        if (i % RSP == 0 && i / RSP < CR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  const int nk = kc / BK;
  using C0 = integral_constant<int, 0>;
  using C1 = integral_constant<int, 1>;
  using C2 = integral_constant<int, 2>;
  // Step kt reads A stage PA = kt % 2 and W stage PW = kt % 3, its sub-step
  // 0 fragments already in register set 0, and has one barrier, in the
  // middle:
  //   sub-step 0's MFMAs run with sub-step 1's fragment reads and the copies
  //   of W slice kt+2 into stage (kt+2) % 3 among them (that stage's slice,
  //   kt-1, was last read before step kt-1's barrier);
  //   wait for the copies of A and W slice kt+1 (all copies but the NCPW
  //   newest, W slice kt+2 -- vector-memory loads complete in issue order)
  //   and for this wave's LDS reads, then the barrier: every wave is done
  //   reading stage PA, and slice kt+1 is in LDS;
  //   sub-step 1's MFMAs run with the copies of A slice kt+2 into stage PA
  //   and the reads of step kt+1's sub-step 0 fragments among them.
  // So a fragment read is always a sub-step ahead of its MFMAs, the barrier
  // waits on nothing the MFMAs need, and an A copy has about a step to land,
  // a W copy a step and a half.
  // The W and A copies go into different halves of the step, spread over
  // each.  Past the last slice the copies repeat slice nk - 1 into a stage
  // nobody reads again, so every step issues the same copies and waits the
  // same count; the wait before the epilogue covers the last of them.
  auto step = [&](int kt, auto pa, auto pw) {
    constexpr int PA = decltype(pa)::value, PW = decltype(pw)::value;
    u32x4 *a = SA(pa), *w = SW(pw);
    const int k2 = min(kt + 2, nk - 1);
    u32x4 *wn = SW(integral_constant<int, (PW + 2) % 3>{});
    phase(C0{}, a, w, 1, integral_constant<int, NCPW>{}, [&](int j) { copy_w1(k2, wn, j); });
    // s_waitcnt vmcnt(NCPW) expcnt(7) lgkmcnt(0), then the barrier
    __builtin_amdgcn_s_waitcnt((NCPW & 15) | (7 << 4) | ((NCPW >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    phase(C1{}, SA(integral_constant<int, PA ^ 1>{}), SW(integral_constant<int, (PW + 1) % 3>{}), 0,
          integral_constant<int, NCPA>{}, [&](int j) { copy_a1(k2, a, j); });
  };
  // slices 0 and 1 of both operands, in that order; wait for slice 0 (all
  // but the NCPA + NCPW newest copies)
#pragma unroll
  for (int j = 0; j < NCPA; ++j) copy_a1(0, sA0, j);
#pragma unroll
  for (int j = 0; j < NCPW; ++j) copy_w1(0, sW0, j);
#pragma unroll
  for (int j = 0; j < NCPA; ++j) copy_a1(min(1, nk - 1), sA1, j);
#pragma unroll
  for (int j = 0; j < NCPW; ++j) copy_w1(min(1, nk - 1), sW1, j);
  constexpr int NPRO = NCPA + NCPW;
  __builtin_amdgcn_s_waitcnt((NPRO & 15) | (7 << 4) | ((NPRO >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  fload(sA0, sW0, 0, 0);
  // groups of six steps (the stage pattern's period); the last group skips
  // the steps past nk whole, a uniform branch.  (Six unguarded steps plus a
  // separate tail of up to five steps make the compiler spill.)
  for (int kt = 0; kt < nk; kt += 6) {
    step(kt, C0{}, C0{});
    if (kt + 1 < nk) step(kt + 1, C1{}, C1{});
    if (kt + 2 < nk) step(kt + 2, C0{}, C2{});
    if (kt + 3 < nk) step(kt + 3, C1{}, C0{});
    if (kt + 4 < nk) step(kt + 4, C0{}, C1{});
    if (kt + 5 < nk) step(kt + 5, C1{}, C2{});
  }
  if constexpr (EPI == EPI_QKV) {
    // the q / k tiles' RoPE rows are loaded while the last copies land; every
    // copy has landed (vmcnt(0) expcnt(7) lgkmcnt(0)) and every fragment read
    // is done before the epilogue reuses the stages
    RopeRows<BM, THREADS> rope;
    if ((tn * BN) / g.H < 2) rope.load(g, m0, tid);
    __builtin_amdgcn_s_waitcnt(7 << 4);
    __syncthreads();
    qkv_epilogue16<BM, THREADS, NT, NW>(g, m0, tn * BN, wm * WT, tn * BN + wn * WF, acc, tid,
                                        LdsObjs<4, BM * 8>{sA0, sA1, sW0, sW1}, rope);
    return;
  }
  // the other epilogues do not use the LDS, but the last steps' repeated
  // copies land before the workgroup gives its LDS up
  __builtin_amdgcn_s_waitcnt(7 << 4);
  const int h4 = 4 * kq;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int m = m0 + wm * WT + 16 * t + fr;
    if (m >= g.M) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      // fragments 0, 1 hold the gate rows of outputs +0..15, +16..31, and
      // fragments 2, 3 the up rows of the same outputs
#pragma unroll
      for (int f = 0; f < 2; ++f)
        store4_swiglu(g, m, tn * (BN / 2) + wn * (WF / 2) + 16 * f + h4, acc[f][t], acc[f + 2][t]);
    } else if (split) {
      float *prow = g.part + ((size_t)kchunk * g.M + m) * g.N;
#pragma unroll
      for (int f = 0; f < NW; ++f) *(f32x4 *)(prow + tn * BN + wn * WF + 16 * f + h4) = acc[f][t];
    } else {
#pragma unroll
      for (int f = 0; f < NW; ++f) store4<EPI>(g, m, tn * BN + wn * WF + 16 * f + h4, acc[f][t]);
    }
  }
}
