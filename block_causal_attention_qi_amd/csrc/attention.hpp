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
// Per workgroup: 32 queries per wave, 8 waves (two per SIMD) or, for small
// images, 4 (one per SIMD); key tiles of 64 copied global -> LDS directly and
// double buffered.  VALU work interleaved among a wave's own MFMAs hides about
// two thirds of its issue time behind them (measured on MI355X; an
// exponential leaves about 1.1 ns exposed), so each wave is software pipelined
// over three tiles: the softmax of tile t runs between the score MFMAs of
// tile t+1 and the PV MFMAs of tile t-1, a few VALU instructions per MFMA.
// MFMA 32x32x16 bf16.
// S^T = K Q^T: the A operand takes the tile's K rows in the order
// kappa(i) = 16*(i/16) + 8*((i/4)&1) + 4*((i/8)&1) + (i&3), which leaves each
// lane holding 8 CONSECUTIVE keys of one query per 16-key step.  Those
// exponentiated scores, packed to bf16, are directly the B operand of
// O^T = V^T P^T, whose A operand is then one contiguous 16-byte read of a V^T
// row.  V is consumed as V^T [heads][128][Tp], which the QKV epilogue writes.
// Softmax statistics are fp32 in the log2 domain (scores enter exp2 through
// one FMA with the folded scale); each query's 64 scores of a tile are split
// over two lanes (l and l^32).  The running sum adds the bf16-rounded
// probabilities (the values the PV product multiplies), two per dot2.  The
// running max is raised only when a tile's max exceeds it by more than 8 (a
// factor of 256), so the accumulator rescale is rare; the probabilities then
// stay below 2^8, far from fp32 or bf16 overflow, and the final division by
// the running sum cancels the choice exactly in real arithmetic.
#pragma once

#include <type_traits>

#include "common.hpp"

#include "attention_args.hpp"


// key (within a 32-key block) fed by A-operand row i, so that output row
// 8j + 4h + r holds key 16*(j>>1) + 8h + 4*(j&1) + r
QI_DEV int kappa(int i) { return ((i >> 4) << 4) + (((i >> 2) & 1) << 3) + (((i >> 3) & 1) << 2) + (i & 3); }

// Schedule of one 16-read / 16-MFMA phase: each LDS fragment read is issued
// two MFMAs ahead of the one that consumes it.
QI_DEV void interleave_reads_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
  for (int i = 0; i < 14; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

// max of x over lanes l and l ^ 32: v_permlane32_swap of x with itself leaves
// x[l % 32] in one result and x[l % 32 + 32] in the other, in every lane (a
// VALU op; a shuffle through ds_bpermute would also wait for every LDS read
// in flight)
QI_DEV float max_over_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// sum += lo + hi of a packed bf16 pair, in fp32
QI_DEV float add_bf16x2(uint32_t pair, float sum) {
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, sum, false);
}

template <int WAVES>
__global__ __launch_bounds__(attn::Shape<WAVES>::THREADS, 1) void block_causal_attn_kernel(const AttnBatch ab) {
  using namespace attn;
  constexpr int BQ = Shape<WAVES>::BQ, THREADS = Shape<WAVES>::THREADS, NLD = Shape<WAVES>::NLD;
  // Double buffers as four separate objects, always indexed by a constant:
  // the compiler then knows that a copy into one buffer does not alias reads
  // of the other and does not make those reads wait for the copy.
  __shared__ u32x4 sK0[BKV * 16], sK1[BKV * 16];  // [key][16 chunks of 8 d], chunk c at c ^ (key & 15)
  __shared__ u32x4 sV0[128 * 8], sV1[128 * 8];    // [d][8 chunks of 8 keys], chunk c at c ^ ((d >> 1) & 7)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
  // L2); renumber them so that each XCD works through whole heads, whose
  // query tiles then stream the same K/V tiles at about the same time.
  // (grid.y enumerates branch-major (branch, head) pairs)
  const int tiles_per_head = gridDim.x, G = gridDim.x * gridDim.y;
  int wg = blockIdx.x + gridDim.x * blockIdx.y;
  if ((G & 7) == 0) wg = (wg & 7) * (G >> 3) + (wg >> 3);
  const int head_c = wg / tiles_per_head;
  int qt = wg - head_c * tiles_per_head;
  const int branch = head_c >= ab.br[0].heads ? 1 : 0;
  const AttnArgs a = branch ? ab.br[1] : ab.br[0];
  if (a.skip && *a.skip) return;
  const int head = head_c - branch * a.heads;
  const bool img = qt < a.n_img_qt;
  if (!img) qt -= a.n_img_qt;
  const int q0 = qt * BQ;
  const int wq0 = q0 + wave * 32;  // this wave's first query
  const int seg_q = img ? a.N : a.L;
  const int qrow = wq0 + l32;
  const u16 *Q = (img ? a.q_i : a.q_t) + (size_t)head * seg_q * 128;

  // B operand of S^T: Q[q][16 ds + 8 h .. +8] for this lane's query
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

  // Tiles are copied global -> LDS directly (no register staging): lane l of
  // a wave-wide copy lands at 16 l past the wave's base, so the swizzle is
  // applied on the global side by choosing which chunk each lane fetches.
  // The copies are buffer loads over one resource per segment and operand
  // (this head's K [len][128], V^T [128][ldv]): each lane's offset inside a
  // tile is fixed and precomputed.  For K the tile's first key is added to
  // that per-lane offset, which the buffer's range check covers, so K rows
  // past the segment read as zeros and never past the caller's buffer
  // (masked below in any case); a V^T tile is always inside its row
  // (ldv >= key0 + 64), so its first key enters as the uniform scalar offset.
  constexpr int RSRC_FLAGS = 0x00020000;  // raw buffer, 32-bit dwords
  const __amdgpu_buffer_rsrc_t rk_t = __builtin_amdgcn_make_buffer_rsrc((void *)Kt, (short)0, a.L * 256, RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rk_i = __builtin_amdgcn_make_buffer_rsrc((void *)Ki, (short)0, a.N * 256, RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rv_t =
      __builtin_amdgcn_make_buffer_rsrc((void *)Vtt, (short)0, 256 * a.ldv_t, RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rv_i =
      __builtin_amdgcn_make_buffer_rsrc((void *)Vti, (short)0, 256 * a.ldv_i, RSRC_FLAGS);
  int koff[NLD], voff_t[NLD], voff_i[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int i = (j * WAVES + wave) * 64 + lane;
    const int kr = i >> 4, kc = (i & 15) ^ (kr & 15);  // K row kr of the tile, chunk kc
    koff[j] = (kr * 128 + kc * 8) * 2;
    const int vr = i >> 3, vc = (i & 7) ^ ((vr >> 1) & 7);  // V^T row vr, chunk vc
    voff_t[j] = (vr * a.ldv_t + vc * 8) * 2;
    voff_i[j] = (vr * a.ldv_i + vc * 8) * 2;
  }
  auto lds_ptr = [](u32x4 *p) { return (__attribute__((address_space(3))) void *)p; };
  // copy instruction j of K / V^T tile t into buffer B
  auto copy_k1 = [&](int t, auto B, int j) {
    u32x4 *sk = B.value ? sK1 : sK0;
    const bool tx = t < nt_t;
    const int key0 = (tx ? t : t - nt_t) * BKV;
#if __HIP_DEVICE_COMPILE__  // the host pass cannot resolve this builtin in a template
    __builtin_amdgcn_raw_ptr_buffer_load_lds(tx ? rk_t : rk_i, lds_ptr(sk + (j * WAVES + wave) * 64), 16,
                                             koff[j] + key0 * 256, 0, 0, 0);
#endif
  };
  auto copy_v1 = [&](int t, auto B, int j) {  // in bounds: ldv >= key0 + 64
    u32x4 *sv = B.value ? sV1 : sV0;
    const bool tx = t < nt_t;
    const int key0 = (tx ? t : t - nt_t) * BKV;
#if __HIP_DEVICE_COMPILE__
    __builtin_amdgcn_raw_ptr_buffer_load_lds(tx ? rv_t : rv_i, lds_ptr(sv + (j * WAVES + wave) * 64), 16,
                                             tx ? voff_t[j] : voff_i[j], key0 * 2, 0, 0);
#endif
  };
  auto copy_k = [&](int t, auto B) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) copy_k1(t, B, j);
  };
  auto copy_v = [&](int t, auto B) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) copy_v1(t, B, j);
  };
  // V^T columns past the segment's end (padding, any bit pattern) become exact
  // zeros, so that their zero probabilities contribute exact zeros.  Only the
  // segment's last tile has them; the caller brackets this with barriers.
  auto zero_v_tail = [&](int t, auto B) {
    const bool tx = t < nt_t;
    const int key0 = (tx ? t : t - nt_t) * BKV;
    const int valid = (tx ? a.L : a.N) - key0;
    if (valid >= BKV) return;
    const int npad = BKV - valid;
    u16 *sv = (u16 *)(B.value ? sV1 : sV0);
    for (int i = tid; i < 128 * npad; i += THREADS) {
      const int vr = i / npad, col = valid + i % npad;
      sv[(vr * 8 + ((col >> 3) ^ ((vr >> 1) & 7))) * 8 + (col & 7)] = 0;
    }
  };
  auto v_tail = [&](int t) {
    const bool tx = t < nt_t;
    return ((tx ? t : t - nt_t) + 1) * BKV > (tx ? a.L : a.N);
  };

  // K row this lane feeds to the S^T MFMA in each 32-key block
  const int krow_l = kappa(l32);
  const int vsw = (l32 >> 1) & 7;
  const float c = a.scale_log2;

  // S^T for 64 keys (2 blocks of 32) x this wave's 32 queries from sK[b]
  auto scores = [&](auto B, f32x16 *s) {
    const u32x4 *sk = B.value ? sK1 : sK0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kr = kb * 32 + krow_l;
        const u32x4 ka = sk[kr * 16 + ((2 * ds + h) ^ (kr & 15))];
        s[kb] = mfma32x32x16(ka, qreg[ds], s[kb]);
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[d][e] = 0.f;

  // Software pipeline over three tiles: iteration t exponentiates the scores
  // of tile t between the score MFMAs of tile t+1 and the PV MFMAs of tile
  // t-1, so the softmax's VALU work is spread over all 32 MFMAs of an
  // iteration.  K runs two tiles ahead in LDS: iteration t copies K(t+2) into
  // sK[t&1], whose K(t) was consumed in iteration t-1.  V(t) is copied in
  // iteration t into sV[t&1] (its V(t-2) was consumed in iteration t-1) and
  // consumed in iteration t+1.  Their copy instructions, V first, go among
  // the first 16 MFMA slots (issued together at the iteration's start, they
  // held the wave's first MFMAs back: 2% more attention time); past the last
  // tile the K copy repeats that tile into the buffer nobody reads again.
  // The compiler waits for the copies before the barrier that ends the
  // iteration.  The accumulators take tile t-1's PV product
  // in tile t-1's base and are rescaled to tile t's base after it, so the
  // arithmetic is the same sequence as rescale-then-accumulate per tile.
  constexpr std::integral_constant<int, 0> B0{};
  constexpr std::integral_constant<int, 1> B1{};
  constexpr std::false_type NO_PV{};
  constexpr std::true_type PV{};
  copy_k(0, B0);
  if (ntiles > 1) copy_k(1, B1);
  __syncthreads();
  // Scores and bf16 probabilities of consecutive tiles alternate between two
  // register sets chosen by the tile's parity (a constant in each unrolled
  // iteration), so no iteration copies one tile's state into the other's.
  f32x16 sA[2], sB[2];  // scores of even / odd tiles
  u32x4 pA[4], pB[4];   // bf16 probabilities of even / odd tiles (PV's B operand)
  scores(B0, sA);
  __syncthreads();  // sK0 is overwritten next

  // O^T[d][q] += V^T[d][16 c4 + 8h .. +8] P^T with V from sV[B]
  auto pv = [&](auto B, const u32x4 *pb) {
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int vr = db * 32 + l32;
        const u32x4 va = (B.value ? sV1 : sV0)[vr * 8 + ((2 * c4 + h) ^ vsw)];
        oacc[db] = mfma32x32x16(va, pb[c4], oacc[db]);
      }
    }
  };

  // one iteration; B = t & 1 as a constant; HAS_PV: tile t-1 exists
  auto iteration = [&](int t, auto B, auto HAS_PV) {
    constexpr std::integral_constant<int, 1 - B.value> NB{};
    f32x16(&s_cur)[2] = B.value ? sB : sA;
    f32x16(&s_next)[2] = B.value ? sA : sB;
    u32x4(&pb)[4] = B.value ? pB : pA;
    const u32x4(&pb_prev)[4] = B.value ? pA : pB;
    const int tk = min(t + 2, ntiles - 1);  // past the end: a copy nobody reads

    // element e of block kb holds key key0 + 32 kb + 16 (e >> 3) + 8 h + (e & 7)
    const bool tx = t < nt_t;
    const int key0 = (tx ? t : t - nt_t) * BKV;
    const int klen = tx ? a.L : a.N;
    const bool causal = !img;
    if ((key0 + BKV > klen) || (causal && key0 + BKV - 1 > wq0)) {
      // keys at or past lim are masked: the segment's end, and for text
      // queries every key after the query (block-causal inside the text)
      const int lim = min(klen, causal ? qrow + 1 : klen) - key0 - 8 * h;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * kb + 16 * (e >> 3) + (e & 7) >= lim) s_cur[kb][e] = -INFINITY;
    }

    // 32 MFMA slots: even slots run the score MFMAs of tile t+1 (from
    // sK[b^1]), odd slots the PV MFMAs of tile t-1 (from sV[b^1]); each slot's
    // LDS fragment is read two slots ahead.  The softmax of tile t is cut into
    // pieces placed between the slots, and sched_barrier keeps each slot's
    // instructions together.
    const u32x4 *sk = NB.value ? sK1 : sK0;
    const u32x4 *sv = NB.value ? sV1 : sV0;
    auto frag = [&](int i) -> u32x4 {
      const int j = i >> 1;
      if ((i & 1) == 0) {
        const int ds = j >> 1, kr = (j & 1) * 32 + krow_l;
        return sk[kr * 16 + ((2 * ds + h) ^ (kr & 15))];
      }
      const int c4 = j >> 2, vr = (j & 3) * 32 + l32;
      return sv[vr * 8 + ((2 * c4 + h) ^ vsw)];
    };
    u32x4 fr[3];
    fr[0] = frag(0);
    if constexpr (HAS_PV.value) fr[1] = frag(1);
    float m4[4], mx = 0.f, alpha = 1.f, nbase = 0.f;
    bool raise = false;
    float psum[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      // this iteration's copies, V(t) first, spread over the first 16 slots
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        if (i == (16 / (2 * NLD)) * j) copy_v1(t, B, j);
        if (i == (16 / (2 * NLD)) * (NLD + j)) copy_k1(tk, B, j);
      }
      const bool slot = HAS_PV.value || (i & 1) == 0;
      if (i + 2 < 32 && (HAS_PV.value || ((i + 2) & 1) == 0)) fr[(i + 2) % 3] = frag(i + 2);
      if (slot) {
        const int j = i >> 1;
        if ((i & 1) == 0) {
          const int kb = j & 1;
          if (j < 2)
            s_next[kb] = mfma32x32x16(fr[i % 3], qreg[j >> 1], f32x16{});
          else
            s_next[kb] = mfma32x32x16(fr[i % 3], qreg[j >> 1], s_next[kb]);
        } else {
          oacc[j & 3] = mfma32x32x16(fr[i % 3], pb_prev[j >> 2], oacc[j & 3]);
        }
      }
      // the slot's softmax piece issues at raised wave priority, so that the
      // SIMD's other wave does not hold it back while this wave's MFMA runs
      // (measured on MI355X: 2-4% less attention time than without)
      __builtin_amdgcn_s_setprio(1);
      // softmax pieces
      if (i < 4) {
        // tile max over this lane's 32 scores: a shallow tree of 3-way maxes
        const f32x16 &s4 = s_cur[i >> 1];
        const int e0 = 8 * (i & 1);
        m4[i] = fmaxf(fmaxf(fmaxf(s4[e0], s4[e0 + 1]), s4[e0 + 2]), fmaxf(fmaxf(s4[e0 + 3], s4[e0 + 4]), s4[e0 + 5]));
        m4[i] = fmaxf(fmaxf(m4[i], s4[e0 + 6]), s4[e0 + 7]);
      } else if (i == 4) {
        mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        mx = max_over_halves(mx) * c;  // with the partner lane's
      } else if (i == 5) {
        // raise the running max only past the slack; only a raised max
        // costs a rescale of the accumulators
        raise = mx > m_run + RESCALE_SLACK;
        if (raise) {
          alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
          m_run = mx;
        }
        nbase = m_run == -INFINITY ? 0.f : -m_run;
      } else {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (6 + (u * 26) / 16 != i) continue;
          // probabilities of keys 16 c4 + 8 h + 2 k, +1 (c4 = 2 kb + cc)
          const int kb = u >> 3, cc = (u >> 2) & 1, k = u & 3, e = 8 * cc + 2 * k;
          const uint32_t w = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[kb][e], c, nbase)),
                                         __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[kb][e + 1], c, nbase)));
          pb[2 * kb + cc][k] = w;
          psum[k & 1] = add_bf16x2(w, psum[k & 1]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run = l_run * alpha + (psum[0] + psum[1]);
    // keep the exponentials between the MFMAs (the compiler would otherwise
    // sink them past the barrier to their use in the next iteration)
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(pb[i]));
    asm volatile("" : "+v"(l_run));

    // tile t-1 is in the accumulators: move them to tile t's base
    if (__any(raise)) {
#pragma unroll
      for (int d = 0; d < 4; ++d) oacc[d] *= alpha;
    }
    __syncthreads();
    if (v_tail(t)) {
      zero_v_tail(t, B);
      __syncthreads();
    }
  };
  iteration(0, B0, NO_PV);
  for (int t = 1; t < ntiles; t += 2) {
    iteration(t, B1, PV);
    if (t + 1 < ntiles) iteration(t + 1, B0, PV);
  }
  // the last tile's PV product
  if ((ntiles - 1) & 1) {
    pv(B1, pB);
    interleave_reads_mfma();
  } else {
    pv(B0, pA);
    interleave_reads_mfma();
  }

  const float l = l_run + __shfl_xor(l_run, 32, 64);
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
