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
// bf16 MFMA count, far above the fp32 MFMA rate.  The kernel that produces a
// matmul input (the RMSNorms, attention, the SwiGLU epilogue) writes it as the
// three planes [3][rows][cols] bf16 once, and the GEMMs copy the planes
// straight into LDS.  The attention (small: L <= 512 tokens) runs on the fp32
// MFMA 32x32x2 directly.
#pragma once

#include "common.hpp"
#include "gemm.hpp"

namespace enc {
constexpr int BM = 64, BN = 128, BK = 32, THREADS = 256, NP = 3;
constexpr int FS = 2;                          // wave tile 32 tokens x 64 W rows
constexpr int NST = 4;                         // stages in the LDS ring
constexpr int A_SLOTS = NP * BM * 4;           // 16-byte slots of a stage's three A planes
constexpr int W_SLOTS = BN * 4;                // of its W slice
constexpr int ST_SLOTS = A_SLOTS + W_SLOTS;    // 20 KB per stage
constexpr int CA = A_SLOTS / THREADS, CW = W_SLOTS / THREADS;  // copies per thread and stage (3, 2)
}  // namespace enc

// the same split of 4 fp32 values, as three 8-byte plane entries
QI_DEV void split3x4(const f32x4 v, u32x2 &p0, u32x2 &p1, u32x2 &p2) {
#pragma unroll
  for (int e = 0; e < 4; e += 2) {
    const uint32_t a = pack_bf16x2(v[e], v[e + 1]);
    const float r0 = v[e] - bf16_to_f32((u16)(a & 0xFFFF)), r1 = v[e + 1] - bf16_to_f32((u16)(a >> 16));
    const uint32_t b = pack_bf16x2(r0, r1);
    const uint32_t c = pack_bf16x2(r0 - bf16_to_f32((u16)(b & 0xFFFF)), r1 - bf16_to_f32((u16)(b >> 16)));
    p0[e / 2] = a;
    p1[e / 2] = b;
    p2[e / 2] = c;
  }
}

// 4 consecutive fp32 values at [row][col] of a plane triple [3][rows][ld]
QI_DEV void store4_planes(u16 *planes, size_t plane_elems, int ld, int row, int col, f32x4 v) {
  u32x2 p0, p1, p2;
  split3x4(v, p0, p1, p2);
  u16 *q = planes + (size_t)row * ld + col;
  *(u32x2 *)q = p0;
  *(u32x2 *)(q + plane_elems) = p1;
  *(u32x2 *)(q + 2 * plane_elems) = p2;
}

enum EncEpi { ENC_F32 = 0, ENC_RESID = 1, ENC_SWIGLU = 2 };

struct EncGemmArgs {
  const u16 *A;    // [3][M][lda] bf16: the three planes of the fp32 input
  int lda;
  const u16 *W;    // [N][ldw] bf16 (SWIGLU: [2F][ldw], gate rows then up rows)
  int ldw;
  int M, N, K;
  float *C;        // ENC_F32: C[m][n] = acc
  int ldc;
  float *X;        // ENC_RESID: X[m][n] += acc
  int ldx;
  u16 *out;        // ENC_SWIGLU: the planes [3][M][ldo] of out[m][o] = SiLU(gate) * up, o < F
  int ldo, F;
};

// 64 x 128 tile of C = A W^T with A fp32 given as its three bf16 planes:
// four waves (2 x 2, wave tile 32 tokens x 64 W rows), two workgroups per CU.
// A K step of 32 moves 12 KB of planes and an 8 KB W slice, copied global ->
// LDS directly (buffer loads with the LDS flag; lane l of a copy lands 16
// bytes at slot base + l) three steps ahead into a ring of four stages, four
// LDS objects of 20 KB indexed by compile-time constants (the K loop is
// unrolled by 4).  The weights stream from HBM, and with only 421 rows per
// forward each W slice feeds few MFMAs: the copies need the deep ring to hide
// their latency.  A step ends with every copy but the two newest slices'
// landed (vmcnt: loads complete in issue order) and its LDS reads done, then
// the barrier.
// Slot layout per 32-wide row (64 bytes = 4 chunks of 16): chunk c of row r at
// slot r * 4 + (c ^ ((r >> 2) & 3)), so the 16 rows one ds_read_b128 pass
// reads at a fixed chunk land on 16 distinct bank groups.  Copy j of wave w
// fills slots (4 j + w) * 64 .. + 63 of its part: 16 rows (A: plane
// (4 j + w) / 4, rows 16 ((4 j + w) % 4) + lane / 4; W: rows 16 (4 j + w) +
// lane / 4), chunk (lane % 4) ^ ((lane / 16) % 4).  Rows past M read as zero
// (plane 2) or as other planes' rows (planes 0, 1): only outputs of rows past
// M see them, and those are never stored.  Per 16-deep sub-step the MFMAs run
// the planes from the smallest up, so the small terms add into small sums
// first.
template <int EPI>
__global__ __launch_bounds__(enc::THREADS, 2) void enc_gemm_kernel(const EncGemmArgs g) {
  using namespace enc;
  __shared__ u32x4 sS0[ST_SLOTS], sS1[ST_SLOTS], sS2[ST_SLOTS], sS3[ST_SLOTS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int nTM = (g.M + BM - 1) / BM;
  const int nTN = EPI == ENC_SWIGLU ? g.F / (BN / 2) : g.N / BN;
  int tm, tn;
  tile_of(blockIdx.x, nTM, nTN, tm, tn);
  const int m0 = tm * BM;

  const size_t plane_elems = (size_t)g.M * g.lda;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void *)g.A, (short)0, (int)(3 * plane_elems * 2), 0x00020000);
  const int wrows = EPI == ENC_SWIGLU ? 2 * g.F : g.N;
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void *)g.W, (short)0, (int)((size_t)wrows * g.ldw * 2), 0x00020000);
  const int lr = lane >> 2;
  const int cch = (lane & 3) ^ ((lane >> 4) & 3);
  int voff_a[CA], voff_w[CW];
#pragma unroll
  for (int j = 0; j < CA; ++j) {
    const int blk = 4 * j + wave;  // 64-slot block: plane blk / 4, rows 16 (blk % 4) ..
    const int row = 16 * (blk & 3) + lr;
    voff_a[j] = (int)(((size_t)(blk >> 2) * plane_elems + (size_t)(m0 + row) * g.lda + cch * 8) * 2);
  }
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int r = 16 * (4 * j + wave) + lr;  // tile row
    int wr;
    if constexpr (EPI == ENC_SWIGLU)
      wr = tn * (BN / 2) + (r >> 6) * 32 + (r & 31) + ((r >> 5) & 1) * g.F;
    else
      wr = tn * BN + r;
    voff_w[j] = (wr * g.ldw + cch * 8) * 2;
  }
  auto lds_ptr = [](u32x4 *p) { return (__attribute__((address_space(3))) void *)p; };
  auto copy = [&](int kt, u32x4 *st) {
#if __HIP_DEVICE_COMPILE__  // the host pass cannot resolve this builtin in a template
#pragma unroll
    for (int j = 0; j < CA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds_ptr(st + (4 * j + wave) * 64), 16, voff_a[j], kt * BK * 2, 0, 0);
#pragma unroll
    for (int j = 0; j < CW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, lds_ptr(st + A_SLOTS + (4 * j + wave) * 64), 16, voff_w[j],
                                               kt * BK * 2, 0, 0);
#endif
  };
  auto stage = [&](auto i) -> u32x4 * {
    if constexpr (decltype(i)::value == 0) return sS0;
    else if constexpr (decltype(i)::value == 1) return sS1;
    else if constexpr (decltype(i)::value == 2) return sS2;
    else return sS3;
  };

  f32x16 acc[FS];
#pragma unroll
  for (int f = 0; f < FS; ++f)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[f][e] = 0.f;

  const int fr = lane & 31, half = lane >> 5;
  const int rowA = wm * 32 + fr, rowW = wn * 64 + fr;
  auto compute = [&](const u32x4 *st) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 fw[FS], fa[NP];
#pragma unroll
      for (int f = 0; f < FS; ++f) {
        const int r = rowW + 32 * f;
        fw[f] = st[A_SLOTS + r * 4 + ((kk * 2 + half) ^ ((r >> 2) & 3))];
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) fa[p] = st[p * BM * 4 + rowA * 4 + ((kk * 2 + half) ^ ((rowA >> 2) & 3))];
#pragma unroll
      for (int p = NP - 1; p >= 0; --p)
#pragma unroll
        for (int f = 0; f < FS; ++f) acc[f] = mfma32x32x16(fw[f], fa[p], acc[f]);
    }
  };
  constexpr int CPS = CA + CW;  // copies per thread and stage
  auto wait_barrier = [&]() {   // s_waitcnt vmcnt(2 CPS) expcnt(7) lgkmcnt(0), then the barrier
    __builtin_amdgcn_s_waitcnt(((2 * CPS) & 15) | (7 << 4) | (((2 * CPS) >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  const int nk = g.K / BK;
  // step kt computes stage kt % 4 after copying slice kt+3 into stage
  // (kt+3) % 4, which step kt-1 read (past the last slice the copies repeat
  // slice nk-1 into a stage never read again)
  auto step = [&](int kt, auto S) {
    constexpr int s4 = decltype(S)::value;
    copy(min(kt + 3, nk - 1), stage(std::integral_constant<int, (s4 + 3) % NST>{}));
    compute(stage(S));
    wait_barrier();
  };
  copy(0, sS0);
  copy(min(1, nk - 1), sS1);
  copy(min(2, nk - 1), sS2);
  wait_barrier();
  int kt = 0;
  for (; kt + 4 <= nk; kt += 4) {
    step(kt, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
    step(kt + 2, std::integral_constant<int, 2>{});
    step(kt + 3, std::integral_constant<int, 3>{});
  }
  if (kt < nk) step(kt, std::integral_constant<int, 0>{});
  if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>{});
  if (kt + 2 < nk) step(kt + 2, std::integral_constant<int, 2>{});
  __syncthreads();  // every copy has landed before the workgroup ends

  // lane holds, for each block f and j, the 4 consecutive W rows
  // f*32 + 8j + 4*half + 0..3 of token rowA
  const int h4 = 4 * half;
  const int m = m0 + rowA;
  if (m >= g.M) return;
  if constexpr (EPI == ENC_SWIGLU) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 gt = quad(acc[0], j), up = quad(acc[1], j);
      f32x4 y;
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = gt[r] / (1.f + expf(-gt[r])) * up[r];
      store4_planes(g.out, (size_t)g.M * g.ldo, g.ldo, m, tn * (BN / 2) + wn * 32 + 8 * j + h4, y);
    }
  } else {
#pragma unroll
    for (int f = 0; f < FS; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = tn * BN + wn * 64 + f * 32 + 8 * j + h4;
        const f32x4 v = quad(acc[f], j);
        if constexpr (EPI == ENC_F32) {
          *(f32x4 *)(g.C + (size_t)m * g.ldc + n) = v;
        } else {
          f32x4 *xp = (f32x4 *)(g.X + (size_t)m * g.ldx + n);
          *xp = *xp + v;
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

// out = x * rsqrt(mean(x^2) + eps) * w over rows of H (H % 256 == 0), fp32,
// written as its three bf16 planes [3][rows][H]; one wave per row, four rows
// per workgroup.
__global__ __launch_bounds__(256) void enc_rmsnorm_kernel(const float *x, const float *w, int rows, int H,
                                                          float eps, u16 *out) {
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
    store4_planes(out, (size_t)rows * H, H, r, c, v * inv * gw);
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
// the score registers.  Softmax in fp32 with expf; out O [L][heads * 128] as
// its three bf16 planes [3][L][heads * 128].
__global__ __launch_bounds__(256) void enc_attention_kernel(const float *Q, const float *K, const float *V, u16 *O,
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
  // K/V tiles go through registers one tile ahead: the loads of tile t+1 are
  // in flight while tile t is computed, and land in LDS at the next step
  constexpr int PER = BKV * 32 / 256;  // float4 of K (and of V) per thread per tile
  f32x4 kr[PER], vr[PER];
  auto load_tile = [&](int key0) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + 256 * j, r = i >> 5, c = (i & 31) * 4;
      const int key = min(key0 + r, L - 1);
      kr[j] = *(const f32x4 *)(Kh + (size_t)key * 128 + c);
      vr[j] = *(const f32x4 *)(Vh + (size_t)key * 128 + c);
    }
  };
  load_tile(0);
  for (int key0 = 0; key0 < kend; key0 += BKV) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {  // 32 float4 per row
      const int i = tid + 256 * j, r = i >> 5, c = (i & 31) * 4;
      *(f32x4 *)&sK[r][c] = kr[j];
      // a key masked by causality meets probability 0, and 0 * v must stay 0:
      // non-finite values (only an invalid input makes them) enter as 0
      f32x4 v = vr[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __builtin_isfinite(v[e]) ? v[e] : 0.f;
      *(f32x4 *)&sV[r][c] = v;
    }
    __syncthreads();
    if (key0 + BKV < kend) load_tile(key0 + BKV);
    if (key0 > wq0 + 31) continue;  // every key of the tile is after every query of this wave
    f32x16 s = {};
#pragma unroll
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
    const int ld = heads * 128;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store4_planes(O, (size_t)L * ld, ld, qrow, head * 128 + 4 * h + 32 * d + 8 * j, quad(oacc[d], j) * inv);
  }
}
