// Kernels of the text encoder (the Qwen3-VL-8B text stack of the port page's
// pieces table: GQA 32:8, q_norm + k_norm, 1-D RoPE theta 5e6, causal; bf16
// weights with fp32 compute, which the page's "<|im_start|> tokens need fp32
// compute" paragraph shows to be required).
//
// fp32 compute with bf16 MFMAs: every activation entering a matmul is fp32,
// every weight is exactly a bf16 value.  An fp32 value a splits exactly into
// three bf16 values a = a0 + a1 + a2 (a0 = bf16(a), a1 = bf16(a - a0),
// a2 = a - a0 - a1; each remainder is exact in fp32 and the last has at most 8
// significant bits), and each product a_p * w of two bf16 values is exact in
// the MFMA's fp32 accumulation.  So one 32x32x16 bf16 MFMA per plane gives the
// fp32 product sum (up to the order of the fp32 additions) at three times the
// bf16 MFMA count, far above the fp32 MFMA rate.  The attention (small: L <=
// 512 tokens) runs on the fp32 MFMA 32x32x2 directly.
#pragma once

#include "common.hpp"
#include "gemm.hpp"

namespace enc {
constexpr int BM = 128, BN = 128, BK = 64, THREADS = 256, NP = 3;
constexpr int TS = 2, FS = 2;  // wave tile 64 tokens x 64 W rows
}  // namespace enc

// exact split of 8 fp32 values into three planes of 8 bf16 (16 bytes each)
QI_DEV void split3(const f32x4 lo, const f32x4 hi, u32x4 &p0, u32x4 &p1, u32x4 &p2) {
  float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  float r1[8], r2[8];
  uint32_t a[4], b[4], c[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    a[e / 2] = pack_bf16x2(v[e], v[e + 1]);
    r1[e] = v[e] - bf16_to_f32((u16)(a[e / 2] & 0xFFFF));
    r1[e + 1] = v[e + 1] - bf16_to_f32((u16)(a[e / 2] >> 16));
    b[e / 2] = pack_bf16x2(r1[e], r1[e + 1]);
    r2[e] = r1[e] - bf16_to_f32((u16)(b[e / 2] & 0xFFFF));
    r2[e + 1] = r1[e + 1] - bf16_to_f32((u16)(b[e / 2] >> 16));
    c[e / 2] = pack_bf16x2(r2[e], r2[e + 1]);
  }
  p0 = u32x4{a[0], a[1], a[2], a[3]};
  p1 = u32x4{b[0], b[1], b[2], b[3]};
  p2 = u32x4{c[0], c[1], c[2], c[3]};
}

// SwiGLU with an fp32 output: outf[m][o..o+3] = SiLU(gate) * up
QI_DEV void store4_swiglu_f32(float *outf, int ldo, int m, int o, f32x4 gt, f32x4 up) {
  f32x4 y;
#pragma unroll
  for (int r = 0; r < 4; ++r) y[r] = gt[r] / (1.f + expf(-gt[r])) * up[r];
  *(f32x4 *)(outf + (size_t)m * ldo + o) = y;
}

enum EncEpi { ENC_F32 = 0, ENC_RESID = 1, ENC_SWIGLU = 2 };

struct EncGemmArgs {
  const float *A;  // [M][lda] fp32
  int lda;
  const u16 *W;    // [N][ldw] bf16 (SWIGLU: [2F][ldw], gate rows then up rows)
  int ldw;
  int M, N, K;
  float *C;        // ENC_F32: C[m][n] = acc
  int ldc;
  float *X;        // ENC_RESID: X[m][n] += acc
  int ldx;
  float *out;      // ENC_SWIGLU: out[m][o], o < F
  int ldo, F;
};

// 128 x 128 tile of C = A W^T with A in fp32, four waves (2 x 2), the three
// A planes and the W tile double-buffered in LDS (2 x (3 x 16 + 16) KB), one
// register stage of the next K slice.
template <int EPI>
__global__ __launch_bounds__(enc::THREADS, 1) void enc_gemm_kernel(const EncGemmArgs g) {
  using namespace enc;
  __shared__ u32x4 sA[2][NP][BM * 8];
  __shared__ u32x4 sW[2][BN * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int nTM = (g.M + BM - 1) / BM;
  const int nTN = EPI == ENC_SWIGLU ? g.F / (BN / 2) : g.N / BN;
  int tm, tn;
  tile_of(blockIdx.x, nTM, nTN, tm, tn);
  const int m0 = tm * BM;

  // thread t moves chunk (i & 7) of tile row i >> 3, i = t + 256 j
  constexpr int CJ = BM * 8 / THREADS;  // 4
  const float *pa[CJ];
  const u16 *pw[CJ];
  int slot[CJ];
#pragma unroll
  for (int j = 0; j < CJ; ++j) {
    const int i = tid + THREADS * j;
    const int row = i >> 3, c = i & 7;
    slot[j] = lds_slot(row, c);
    pa[j] = g.A + (size_t)min(m0 + row, g.M - 1) * g.lda + c * 8;  // rows past M: valid, never stored
    int wr;
    if constexpr (EPI == ENC_SWIGLU) {
      const int s = row >> 5;
      wr = tn * (BN / 2) + (s >> 1) * 32 + (row & 31) + (s & 1) * g.F;
    } else {
      wr = tn * BN + row;
    }
    pw[j] = g.W + (size_t)wr * g.ldw + c * 8;
  }
  f32x4 ra[CJ][2];
  u32x4 rw[CJ];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int j = 0; j < CJ; ++j) {
      ra[j][0] = *(const f32x4 *)(pa[j] + k0);
      ra[j][1] = *(const f32x4 *)(pa[j] + k0 + 4);
      rw[j] = *(const u32x4 *)(pw[j] + k0);
    }
  };
  auto lstore = [&](int b) {
#pragma unroll
    for (int j = 0; j < CJ; ++j) {
      u32x4 p0, p1, p2;
      split3(ra[j][0], ra[j][1], p0, p1, p2);
      sA[b][0][slot[j]] = p0;
      sA[b][1][slot[j]] = p1;
      sA[b][2][slot[j]] = p2;
      sW[b][slot[j]] = rw[j];
    }
  };

  f32x16 acc[FS][TS];
#pragma unroll
  for (int f = 0; f < FS; ++f)
#pragma unroll
    for (int t = 0; t < TS; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][t][e] = 0.f;

  const int fr = lane & 31, half = lane >> 5;
  const int nk = g.K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int b = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = kk * 2 + half;
      u32x4 fw[FS];
#pragma unroll
      for (int f = 0; f < FS; ++f) fw[f] = sW[b][lds_slot(wn * 64 + f * 32 + fr, ch)];
      // planes from the smallest up, so the small terms add into small sums first
#pragma unroll
      for (int p = NP - 1; p >= 0; --p) {
        u32x4 fa[TS];
#pragma unroll
        for (int t = 0; t < TS; ++t) fa[t] = sA[b][p][lds_slot(wm * 64 + t * 32 + fr, ch)];
#pragma unroll
        for (int f = 0; f < FS; ++f)
#pragma unroll
          for (int t = 0; t < TS; ++t) acc[f][t] = mfma32x32x16(fw[f], fa[t], acc[f][t]);
      }
    }
    if (kt + 1 < nk) lstore(b ^ 1);
    __syncthreads();
  }

  // lane holds, for each (f, t) block and j, the 4 consecutive W rows
  // f*32 + 8j + 4*half + 0..3 of token t*32 + lane%32
  const int h4 = 4 * half;
#pragma unroll
  for (int t = 0; t < TS; ++t) {
    const int m = m0 + wm * 64 + t * 32 + fr;
    if (m >= g.M) continue;
    if constexpr (EPI == ENC_SWIGLU) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store4_swiglu_f32(g.out, g.ldo, m, tn * (BN / 2) + wn * 32 + 8 * j + h4, quad(acc[0][t], j),
                          quad(acc[1][t], j));
    } else {
#pragma unroll
      for (int f = 0; f < FS; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = tn * BN + wn * 64 + f * 32 + 8 * j + h4;
          const f32x4 v = quad(acc[f][t], j);
          if constexpr (EPI == ENC_F32) {
            *(f32x4 *)(g.C + (size_t)m * g.ldc + n) = v;
          } else {
            f32x4 *xp = (f32x4 *)(g.X + (size_t)m * g.ldx + n);
            *xp = *xp + v;
          }
        }
    }
  }
}

// x[t][:] = embed[ids[t]][:] as fp32 (exact); an id outside the vocabulary
// gives a NaN row (never an out-of-range read).
__global__ __launch_bounds__(256) void enc_embed_kernel(const int *ids, int vocab, const u16 *embed, int H,
                                                        float *x) {
  const int t = blockIdx.x;
  const int id = ids[t];
  if (id >= 0 && id < vocab) {
    for (int c = threadIdx.x; c < H; c += blockDim.x) x[(size_t)t * H + c] = bf16_to_f32(embed[(size_t)id * H + c]);
  } else {
    for (int c = threadIdx.x; c < H; c += blockDim.x) x[(size_t)t * H + c] = __builtin_nanf("");
  }
}

// out = x * rsqrt(mean(x^2) + eps) * w over rows of H (H % 256 == 0), fp32;
// one wave per row, four rows per workgroup.
__global__ __launch_bounds__(256) void enc_rmsnorm_kernel(const float *x, const float *w, int rows, int H,
                                                          float eps, float *out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float *xr = x + (size_t)r * H;
  float ss = 0.f;
  for (int c = lane * 4; c < H; c += 256) {
    const f32x4 v = *(const f32x4 *)(xr + c);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  const float inv = 1.f / sqrtf(ss / (float)H + eps);
  for (int c = lane * 4; c < H; c += 256) {
    const f32x4 v = *(const f32x4 *)(xr + c);
    const f32x4 gw = *(const f32x4 *)(w + c);
    *(f32x4 *)(out + (size_t)r * H + c) = v * inv * gw;
  }
}

// Per (token, head) of the fused projection qkv [L][(heads + 2 kvh) * 128]:
// q and k heads get the per-head RMSNorm (q_norm / k_norm, eps) and the
// rotate-half RoPE of the token's position (feature i pairs with i + 64; lane
// l holds both), v heads are copied.  Out: Q [heads][L][128], K, V [kvh][L][128].
__global__ __launch_bounds__(256) void enc_qk_prep_kernel(const float *qkv, int L, int heads, int kvh,
                                                          const float *qn, const float *kn, const float *cos,
                                                          const float *sin, float eps, float *Q, float *K,
                                                          float *V) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nh = heads + 2 * kvh;
  if (wid >= L * nh) return;
  const int t = wid / nh, hc = wid - t * nh;
  const float *src = qkv + (size_t)t * nh * 128 + hc * 128;
  const float a = src[lane], b = src[lane + 64];
  if (hc >= heads + kvh) {  // v
    float *dst = V + ((size_t)(hc - heads - kvh) * L + t) * 128;
    dst[lane] = a;
    dst[lane + 64] = b;
    return;
  }
  const bool isq = hc < heads;
  const float *nw = isq ? qn : kn;
  const float ss = wave_sum(a * a + b * b);
  const float inv = 1.f / sqrtf(ss / 128.f + eps);
  const float an = a * inv * nw[lane], bn = b * inv * nw[lane + 64];
  const float c = cos[t * 64 + lane], s = sin[t * 64 + lane];
  float *dst = isq ? Q + ((size_t)hc * L + t) * 128 : K + ((size_t)(hc - heads) * L + t) * 128;
  dst[lane] = an * c - bn * s;
  dst[lane + 64] = bn * c + an * s;
}

QI_DEV f32x16 mfma32x32x2f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

namespace enca {
constexpr int WAVES = 4, BQ = 32 * WAVES, BKV = 32;
}

// Causal GQA attention in fp32 on the fp32 MFMA 32x32x2: each wave owns 32
// queries; key tiles of 32 staged in LDS.  S^T = K Q^T contracts d in the
// order lane half h -> features 64 h + s (s = 0..63), so each lane reads 64
// consecutive floats of its query and of a key row.  Output element i of a
// lane (query l % 32) is key kappa(i, h) = 8 (i / 4) + 4 h + i % 4 of the
// tile, and step s of O^T = V^T P^T pairs key kappa(s, 0) (lanes of half 0)
// with kappa(s, 1) (half 1), so the probabilities feed the MFMA straight from
// the score registers.  Softmax in fp32 with expf; out O [L][heads * 128].
__global__ __launch_bounds__(256) void enc_attention_kernel(const float *Q, const float *K, const float *V, float *O,
                                                            int L, int heads, int kvh) {
  using namespace enca;
  // rows padded to 132 floats: a column read by 32 lanes (32 rows) then hits
  // 16 distinct bank groups instead of one
  __shared__ float sK[BKV][132];
  __shared__ float sV[BKV][132];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int head = blockIdx.y, kv = head / (heads / kvh);
  const int q0 = blockIdx.x * BQ, wq0 = q0 + wave * 32;
  const int qrow = wq0 + l32;
  const float *Qh = Q + (size_t)head * L * 128;
  const float *Kh = K + (size_t)kv * L * 128;
  const float *Vh = V + (size_t)kv * L * 128;
  float qreg[64];
  {
    const float *qp = Qh + (size_t)min(qrow, L - 1) * 128 + 64 * h;
#pragma unroll
    for (int s = 0; s < 64; s += 4) {
      const f32x4 v = *(const f32x4 *)(qp + s);
      qreg[s] = v[0]; qreg[s + 1] = v[1]; qreg[s + 2] = v[2]; qreg[s + 3] = v[3];
    }
  }
  const float scale = 1.f / sqrtf(128.f);
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[d][e] = 0.f;
  const int kend = min(q0 + BQ, L);  // keys 0 .. kend-1 reach this workgroup's queries
  for (int key0 = 0; key0 < kend; key0 += BKV) {
    __syncthreads();
    for (int i = tid; i < BKV * 32; i += 256) {  // 32 float4 per row
      const int r = i >> 5, c = (i & 31) * 4;
      const int key = min(key0 + r, L - 1);
      *(f32x4 *)&sK[r][c] = *(const f32x4 *)(Kh + (size_t)key * 128 + c);
      // a key masked by causality meets probability 0, and 0 * v must stay 0:
      // non-finite values (only an invalid input makes them) enter as 0
      f32x4 v = *(const f32x4 *)(Vh + (size_t)key * 128 + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __builtin_isfinite(v[e]) ? v[e] : 0.f;
      *(f32x4 *)&sV[r][c] = v;
    }
    __syncthreads();
    if (key0 > wq0 + 31) continue;  // every key of the tile is after every query of this wave
    f32x16 s = {};
#pragma unroll 16
    for (int j = 0; j < 64; ++j) s = mfma32x32x2f32(sK[l32][64 * h + j], qreg[j], s);
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = key0 + 8 * (e >> 2) + 4 * h + (e & 3);
      const float v = (key <= qrow && key < L) ? s[e] * scale : -INFINITY;
      s[e] = v;
      mx = fmaxf(mx, v);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_run == -INFINITY ? 0.f : expf(m_run - m_new);
    const float base = m_new == -INFINITY ? 0.f : m_new;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s[e] = expf(s[e] - base);
      psum += s[e];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < 4; ++d) oacc[d] *= alpha;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        const int key = 8 * (st >> 2) + 4 * h + (st & 3);
        oacc[d] = mfma32x32x2f32(sV[key][32 * d + l32], s[st], oacc[d]);
      }
  }
  const float inv = 1.f / (l_run + __shfl_xor(l_run, 32, 64));
  if (qrow < L) {
    float *op = O + (size_t)qrow * heads * 128 + head * 128 + 4 * h;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) *(f32x4 *)(op + 32 * d + 8 * j) = quad(oacc[d], j) * inv;
  }
}
