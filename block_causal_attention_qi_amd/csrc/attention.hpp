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
// Per workgroup: 128 queries (4 waves x 32), key tiles of 64 staged through
// LDS (double buffered).  S^T = K Q^T on MFMA 16x16x32 bf16 leaves each lane
// with 4 consecutive keys of one query; those exp'd probabilities are reused
// in registers as the B operand of O^T = V^T P^T by pairing key slots
// {4g..4g+3, 16+4g..16+4g+3} on both operands (a permutation of the MFMA's
// k index, which a dot product does not see).  V is consumed as V^T
// [heads][128][Tp], which the QKV epilogue writes directly.  Softmax
// statistics are fp32, in the log2 domain.
#pragma once

#include "common.hpp"

struct AttnArgs {
  const u16 *q_t, *k_t, *vt_t;  // text segment  (q_t unused when n_txt_qt == 0)
  const u16 *q_i, *k_i, *vt_i;  // image segment
  u16 *o;
  int ldo;                       // heads * 128
  int heads, L, N;
  int ldv_t, ldv_i;              // V^T row strides (>= segment length rounded up to 64)
  int n_img_qt, n_txt_qt;        // query tiles of 128 per head
  int o_img_row0;                // output row of image query 0 (L in a joint pass, else 0)
  float scale_log2;              // log2(e) / sqrt(128)
};

namespace attn {
constexpr int BQ = 128;
constexpr int BKV = 64;
constexpr int THREADS = 256;
}  // namespace attn

__global__ __launch_bounds__(attn::THREADS, 2) void block_causal_attn_kernel(const AttnArgs a) {
  using namespace attn;
  __shared__ u32x4 sK[2][BKV * 16];  // [key][16 chunks of 8 d], chunk c at c ^ (key & 15)
  __shared__ u32x2 sV[2][128 * 16];  // [d][16 chunks of 4 keys], chunk c at c ^ (d & 15)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int head = blockIdx.y;
  int qt = blockIdx.x;
  const bool img = qt < a.n_img_qt;
  if (!img) qt -= a.n_img_qt;
  const int q0 = qt * BQ;
  const int seg_q = img ? a.N : a.L;
  const u16 *Q = (img ? a.q_i : a.q_t) + (size_t)head * seg_q * 128;

  int qrow[2];
  u32x4 qreg[2][4];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    qrow[qs] = q0 + wave * 32 + qs * 16 + l16;
    const int r = min(qrow[qs], seg_q - 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qreg[qs][kk] = *(const u32x4 *)(Q + (size_t)r * 128 + kk * 32 + 8 * grp);
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

  u32x4 rk[4], rv[4];
  auto gload = [&](int t) {
    const bool tx = t < nt_t;
    const u16 *K = tx ? Kt : Ki;
    const u16 *Vt = tx ? Vtt : Vti;
    const int key0 = (tx ? t : t - nt_t) * BKV;
    const int klen = tx ? a.L : a.N;
    const int ldv = tx ? a.ldv_t : a.ldv_i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
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
          uint32_t keep = (k2 < klen ? 0x0000FFFFu : 0u) | (k2 + 1 < klen ? 0xFFFF0000u : 0u);
          v[e] &= keep;
        }
      }
      rv[j] = v;
    }
  };
  auto lstore = [&](int b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + THREADS * j;
      const int kr = i >> 4, kc = i & 15;
      sK[b][kr * 16 + (kc ^ (kr & 15))] = rk[j];
      const int vr = i >> 3, vc = i & 7;
      sV[b][vr * 16 + ((2 * vc) ^ (vr & 15))] = u32x2{rv[j][0], rv[j][1]};
      sV[b][vr * 16 + ((2 * vc + 1) ^ (vr & 15))] = u32x2{rv[j][2], rv[j][3]};
    }
  };

  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f32x4 oacc[8][2];
#pragma unroll
  for (int d = 0; d < 8; ++d)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) oacc[d][qs] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int b = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) gload(t + 1);

    // S^T[key][q] for 64 keys x 32 queries
    f32x4 s[4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) s[ks][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kr = ks * 16 + l16;
        const u32x4 ka = sK[b][kr * 16 + ((kk * 4 + grp) ^ (kr & 15))];
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) s[ks][qs] = mfma16x16x32(ka, qreg[qs][kk], s[ks][qs]);
      }
    }

    const bool tx = t < nt_t;
    const int key0 = (tx ? t : t - nt_t) * BKV;
    const int klen = tx ? a.L : a.N;
    const bool causal = !img;
    const bool need_mask = (key0 + BKV > klen) || (causal && key0 + BKV - 1 > q0 + wave * 32);

    u32x4 pb[2][2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      float mx = -INFINITY;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = s[ks][qs][r] * a.scale_log2;
          if (need_mask) {
            const int key = key0 + ks * 16 + 4 * grp + r;
            const bool ok = key < klen && (!causal || key <= qrow[qs]);
            v = ok ? v : -INFINITY;
          }
          s[ks][qs][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[qs], mx);
      const float base = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run[qs] - base);
      m_run[qs] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = exp2f(s[ks][qs][r] - base);
          s[ks][qs][r] = p;
          psum += p;
        }
      l_run[qs] = l_run[qs] * alpha + psum;
#pragma unroll
      for (int d = 0; d < 8; ++d) oacc[d][qs] *= alpha;
#pragma unroll
      for (int c = 0; c < 2; ++c)
        pb[c][qs] = u32x4{pack_bf16x2(s[2 * c][qs][0], s[2 * c][qs][1]),
                          pack_bf16x2(s[2 * c][qs][2], s[2 * c][qs][3]),
                          pack_bf16x2(s[2 * c + 1][qs][0], s[2 * c + 1][qs][1]),
                          pack_bf16x2(s[2 * c + 1][qs][2], s[2 * c + 1][qs][3])};
    }

    // O^T[d][q] += V^T[d][keys] P^T[keys][q]
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      const int vr = ds * 16 + l16;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x2 lo = sV[b][vr * 16 + ((8 * c + grp) ^ (vr & 15))];
        const u32x2 hi = sV[b][vr * 16 + ((8 * c + 4 + grp) ^ (vr & 15))];
        const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) oacc[ds][qs] = mfma16x16x32(va, pb[c][qs], oacc[ds][qs]);
      }
    }

    if (more) lstore(b ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    float l = l_run[qs];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.f / l;
    if (qrow[qs] < seg_q) {
      const int orow = (img ? a.o_img_row0 : 0) + qrow[qs];
      u16 *op = a.o + (size_t)orow * a.ldo + head * 128 + 4 * grp;
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        const f32x4 v = oacc[ds][qs] * inv;
        *(u32x2 *)(op + ds * 16) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
}
