// Block-causal flash attention for gfx950 (the port page's DiT row: text
// causal over text, image rows see all text and all image keys; the MLX page's
// "Text K/V reuse": text rows never see the image).
//
// One launch covers both segments of every head: grid.x enumerates the image
// query tiles first (they are the heavy ones, L + N keys each) and then the
// text query tiles (causal, <= L keys), grid.y the heads.  Masked key tiles
// are never visited: a text tile walks only the text key tiles up to its
// diagonal.  Keys are always walked in the same order -- text key tiles from
// the text K/V buffer (scratch or the cache), then image key tiles -- so an
// image row computes bit-identical results in a joint pass and in an
// image-only pass that reads the cached text K/V.
//
// Per workgroup: 256 queries (8 waves x 32), key tiles of 64 staged through
// LDS (double buffered), MFMA 32x32x16 bf16 (the full-rate shape on gfx950).
// S^T = K Q^T: the A operand takes the tile's K rows in the order
// kappa(i) = 16*(i/16) + 8*((i/4)&1) + 4*((i/8)&1) + (i&3), which leaves each
// lane holding 8 CONSECUTIVE keys of one query per 16-key step.  Those
// exponentiated scores, packed to bf16, are directly the B operand of
// O^T = V^T P^T, whose A operand is then one contiguous 16-byte read of a V^T
// row.  V is consumed as V^T [heads][128][Tp], which the QKV epilogue writes.
// Softmax statistics are fp32 in the log2 domain; each query's 64 scores of a
// tile are split over two lanes (l and l^32).  The running max is raised only
// when a tile's max exceeds it by more than 8 (a factor of 256), so the
// accumulator rescale is rare; the probabilities then stay below 2^8, far from
// fp32 or bf16 overflow, and the final division by the running sum cancels the
// choice exactly in real arithmetic.
#pragma once

#include "common.hpp"

struct AttnArgs {
  const u16 *q_t, *k_t, *vt_t;  // text segment  (q_t unused when n_txt_qt == 0)
  const u16 *q_i, *k_i, *vt_i;  // image segment
  u16 *o;
  int ldo;                       // heads * 128
  int heads, L, N;
  int ldv_t, ldv_i;              // V^T row strides (>= segment length rounded up to 64)
  int n_img_qt, n_txt_qt;        // query tiles of BQ per head
  int o_img_row0;                // output row of image query 0 (L in a joint pass, else 0)
  float scale_log2;              // log2(e) / sqrt(128)
};

namespace attn {
constexpr int BQ = 256;
constexpr int BKV = 64;
constexpr int THREADS = 512;
constexpr int NLD = BKV * 16 / THREADS;  // 16-byte K (and V^T) chunks per thread per tile
constexpr float RESCALE_SLACK = 8.f;   // log2 units
}  // namespace attn

// key (within a 32-key block) fed by A-operand row i, so that output row
// 8j + 4h + r holds key 16*(j>>1) + 8h + 4*(j&1) + r
QI_DEV int kappa(int i) { return ((i >> 4) << 4) + (((i >> 2) & 1) << 3) + (((i >> 3) & 1) << 2) + (i & 3); }

__global__ __launch_bounds__(attn::THREADS, 1) void block_causal_attn_kernel(const AttnArgs a) {
  using namespace attn;
  __shared__ u32x4 sK[2][BKV * 16];  // [key][16 chunks of 8 d], chunk c at c ^ (key & 15)
  __shared__ u32x4 sV[2][128 * 8];   // [d][8 chunks of 8 keys], chunk c at c ^ ((d >> 1) & 7)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int head = blockIdx.y;
  int qt = blockIdx.x;
  const bool img = qt < a.n_img_qt;
  if (!img) qt -= a.n_img_qt;
  const int q0 = qt * BQ;
  const int seg_q = img ? a.N : a.L;
  const u16 *Q = (img ? a.q_i : a.q_t) + (size_t)head * seg_q * 128;

  // B operand of S^T: Q[q][16 ds + 8 h .. +8] for this lane's query
  const int qrow = q0 + wave * 32 + l32;
  u32x4 qreg[8];
  {
    const int r = min(qrow, seg_q - 1);
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) qreg[ds] = *(const u32x4 *)(Q + (size_t)r * 128 + ds * 16 + 8 * h);
  }

  int nt_t, nt_i;
  if (img) {
    nt_t = (a.L + BKV - 1) / BKV;
    nt_i = (a.N + BKV - 1) / BKV;
  } else {
    nt_t = min(q0 + BQ - 1, a.L - 1) / BKV + 1;
    nt_i = 0;
  }
  const int ntiles = nt_t + nt_i;

  const u16 *Kt = a.k_t + (size_t)head * a.L * 128;
  const u16 *Vtt = a.vt_t + (size_t)head * 128 * a.ldv_t;
  const u16 *Ki = a.k_i + (size_t)head * a.N * 128;
  const u16 *Vti = a.vt_i + (size_t)head * 128 * a.ldv_i;

  u32x4 rk[NLD], rv[NLD];
  auto gload = [&](int t) {
    const bool tx = t < nt_t;
    const u16 *K = tx ? Kt : Ki;
    const u16 *Vt = tx ? Vtt : Vti;
    const int key0 = (tx ? t : t - nt_t) * BKV;
    const int klen = tx ? a.L : a.N;
    const int ldv = tx ? a.ldv_t : a.ldv_i;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int i = tid + THREADS * j;
      const int kr = i >> 4, kc = i & 15;
      const int key = min(key0 + kr, klen - 1);  // rows past the segment: masked below
      rk[j] = *(const u32x4 *)(K + (size_t)key * 128 + kc * 8);
      const int vr = i >> 3, vc = i & 7;
      const int kb = key0 + vc * 8;  // in bounds: ldv >= key0 + 64
      u32x4 v = *(const u32x4 *)(Vt + (size_t)vr * ldv + kb);
      if (kb + 8 > klen) {  // tail of the segment: padding columns become exact zeros
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k2 = kb + 2 * e;
          const uint32_t keep = (k2 < klen ? 0x0000FFFFu : 0u) | (k2 + 1 < klen ? 0xFFFF0000u : 0u);
          v[e] &= keep;
        }
      }
      rv[j] = v;
    }
  };
  auto lstore = [&](int b) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int i = tid + THREADS * j;
      const int kr = i >> 4, kc = i & 15;
      sK[b][kr * 16 + (kc ^ (kr & 15))] = rk[j];
      const int vr = i >> 3, vc = i & 7;
      sV[b][vr * 8 + (vc ^ ((vr >> 1) & 7))] = rv[j];
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[d][e] = 0.f;

  // K row this lane feeds to the S^T MFMA in each 32-key block
  const int krow_l = kappa(l32);
  const int vsw = (l32 >> 1) & 7;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int b = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) gload(t + 1);

    // S^T for 64 keys (2 blocks of 32) x this wave's 32 queries
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kr = kb * 32 + krow_l;
        const u32x4 ka = sK[b][kr * 16 + ((2 * ds + h) ^ (kr & 15))];
        s[kb] = mfma32x32x16(ka, qreg[ds], s[kb]);
      }
    }

    const bool tx = t < nt_t;
    const int key0 = (tx ? t : t - nt_t) * BKV;
    const int klen = tx ? a.L : a.N;
    const bool causal = !img;
    const bool need_mask = (key0 + BKV > klen) || (causal && key0 + BKV - 1 > q0 + wave * 32);

    // element e of block kb holds key key0 + 32 kb + 16 (e >> 3) + 8 h + (e & 7)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = s[kb][e] * a.scale_log2;
        if (need_mask) {
          const int key = key0 + 32 * kb + 16 * (e >> 3) + 8 * h + (e & 7);
          const bool ok = key < klen && (!causal || key <= qrow);
          v = ok ? v : -INFINITY;
        }
        s[kb][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // raise the running max only past the slack; every lane of the wave
    // follows the same rule, and only a raised max costs a rescale
    const bool raise = mx > m_run + RESCALE_SLACK;
    float alpha = 1.f;
    if (raise) {
      alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
      m_run = mx;
    }
    const float base = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
    u32x4 pb[4];  // B operand per 16-key step c4 = 2 kb + c: keys 16 c4 + 8 h .. +8
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = __builtin_amdgcn_exp2f(s[kb][e] - base);
        psum += p[e];
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
        pb[2 * kb + c] = u32x4{pack_bf16x2(p[8 * c], p[8 * c + 1]), pack_bf16x2(p[8 * c + 2], p[8 * c + 3]),
                               pack_bf16x2(p[8 * c + 4], p[8 * c + 5]), pack_bf16x2(p[8 * c + 6], p[8 * c + 7])};
    }
    l_run = l_run * alpha + psum;
    if (__any(raise)) {
#pragma unroll
      for (int d = 0; d < 4; ++d) oacc[d] *= alpha;
    }

    // O^T[d][q] += V^T[d][16 c4 + 8h .. +8] P^T
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int vr = db * 32 + l32;
        const u32x4 va = sV[b][vr * 8 + ((2 * c4 + h) ^ vsw)];
        oacc[db] = mfma32x32x16(va, pb[c4], oacc[db]);
      }
    }

    if (more) lstore(b ^ 1);
    __syncthreads();
  }

  float l = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l;
  if (qrow < seg_q) {
    const int orow = (img ? a.o_img_row0 : 0) + qrow;
    u16 *op = a.o + (size_t)orow * a.ldo + head * 128 + 4 * h;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = quad(oacc[db], j) * inv;
        *(u32x2 *)(op + db * 32 + 8 * j) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
  }
}
