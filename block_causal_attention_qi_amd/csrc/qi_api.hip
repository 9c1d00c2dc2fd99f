// C ABI of the DiT step (include/qi.h): host-side validation, workspace
// carving and the launch sequence of one block and one step.  Everything is
// enqueued on the caller's stream; nothing here synchronises or allocates.
#include <math.h>

#include <cmath>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/qi.h"
#include "attention_args.hpp"
#include "elementwise.hpp"
#include "encoder.hpp"
#include "gemm.hpp"

namespace {

constexpr float kRmsEps = 1e-6f;
constexpr int kMaxL = 512, kMaxN = 16384;

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }
inline int round64(int v) { return (v + 63) & ~63; }
inline bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool dims_ok(const qi_dims *d) {
  if (!d) return false;
  if (d->head_dim != 128) return false;
  if (d->hidden < 256 || d->hidden > 8192 || d->hidden % 256 != 0) return false;
  if (d->heads * 128 != d->hidden) return false;
  if (d->ffn < 64 || d->ffn % 64 != 0 || d->ffn > 65536) return false;
  if (d->txt_dim < 256 || d->txt_dim % 256 != 0 || d->txt_dim > 8192) return false;
  if (d->n_blocks < 1 || d->n_blocks > 256) return false;
  return true;
}

// Workspace of one joint pass over T = L + N rows (an image-only pass uses a
// prefix of each buffer).
struct Layout {
  size_t x, mod, tn, h, q_t, k_t, vt_t, q_i, k_i, vt_i, o, a, part, total;
};

// K-split of the residual GEMMs (O-proj, K = H; down, K = F) for a render of N
// image tokens.  A small image gives the whole-K 128 x 128 tiles too few
// workgroups for 256 CUs (160 at N = 576), so their K is cut into chunks
// whose partial sums resid_reduce_kernel adds in order.  The choice depends
// on N only, so both passes of a render and both CFG branches split alike.
constexpr int kSplitMaxN = 1024;
int ksplit_for(int N, int K, int want) {
  if (N > kSplitMaxN) return 1;
  int s = want;
  while (s > 1 && K % (s * gemm::BK) != 0) --s;
  return s;
}
int ksplit_o(const qi_dims &d, int N) { return ksplit_for(N, d.hidden, 2); }
int ksplit_down(const qi_dims &d, int N) { return ksplit_for(N, d.ffn, 3); }
size_t part_bytes(const qi_dims &d, int N, size_t rows) {
  const int s = std::max(ksplit_o(d, N), ksplit_down(d, N));
  return s > 1 ? (size_t)s * rows * d.hidden * 4 : 0;
}

Layout layout(const qi_dims &d, int L, int N) {
  const size_t H = d.hidden, F = d.ffn, D = d.txt_dim, T = (size_t)L + N;
  const size_t Lp = round64(L), Np = round64(N);
  Layout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  l.x = take(T * H * 4);
  l.mod = take(2 * 4 * H * 4);
  l.tn = take((size_t)L * D * 2);
  l.h = take(T * H * 2);
  l.q_t = take((size_t)L * H * 2);
  l.k_t = take((size_t)L * H * 2);
  l.vt_t = take(H * Lp * 2);
  l.q_i = take((size_t)N * H * 2);
  l.k_i = take((size_t)N * H * 2);
  l.vt_i = take(H * Np * 2);
  l.o = take(T * H * 2);
  l.a = take(T * F * 2);
  l.part = take(part_bytes(d, N, T));
  l.total = off;
  return l;
}

// Workspace of one true-CFG image-only pass: two branches of N image rows
// (no text rows), each with its own Q, K, V^T.
Layout layout_cfg(const qi_dims &d, int N) {
  const size_t H = d.hidden, F = d.ffn, R = 2 * (size_t)N, Np = round64(N);
  Layout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  l.x = take(R * H * 4);
  l.mod = take(2 * 4 * H * 4);
  l.tn = l.q_t = l.k_t = l.vt_t = 0;  // unused
  l.h = take(R * H * 2);
  l.q_i = take(R * H * 2);
  l.k_i = take(R * H * 2);
  l.vt_i = take(2 * H * Np * 2);
  l.o = take(R * H * 2);
  l.a = take(R * F * 2);
  l.part = take(part_bytes(d, N, R));
  l.total = off;
  return l;
}

size_t slot_elems(const qi_dims &d, int L) {
  return (size_t)d.heads * 128 * ((size_t)L + round64(L));
}

qi_status last_launch() { return hipGetLastError() == hipSuccess ? QI_OK : QI_ERR_HIP; }

// ---------------------------------------------------------------- kernel timing
// Optional per-kernel timing: while enabled, every launch is bracketed by two
// events from a pool created by qi_timing_begin, on the launch's own stream.
struct KernelTimer {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<int> kinds;  // kind of each recorded pair
  size_t dropped = 0;
};
KernelTimer g_timer;

struct TimedLaunch {
  hipStream_t s;
  int kind;
  int idx = -1;
  TimedLaunch(int k, hipStream_t st) : s(st), kind(k) {
    std::lock_guard<std::mutex> g(g_timer.mu);
    if (!g_timer.on) return;
    const size_t pair = g_timer.kinds.size();
    if (2 * pair + 1 >= g_timer.pool.size()) {
      ++g_timer.dropped;
      return;
    }
    idx = (int)pair;
    g_timer.kinds.push_back(kind);
    (void)hipEventRecord(g_timer.pool[2 * pair], s);
  }
  ~TimedLaunch() {
    if (idx < 0) return;
    std::lock_guard<std::mutex> g(g_timer.mu);
    (void)hipEventRecord(g_timer.pool[2 * idx + 1], s);
  }
};

#define QI_TRY(expr)               \
  do {                             \
    qi_status s__ = (expr);        \
    if (s__ != QI_OK) return s__;  \
  } while (0)

// The register-staged 128 x 128 kernel, for operands past 32-bit buffer offsets.
template <int EPI, int BM, int BN>
void launch_gemm_tile(const GemmArgs &g, hipStream_t s) {
  const int nTM = (g.M + BM - 1) / BM;
  const int nTN = EPI == EPI_SWIGLU ? g.F / (BN / 2) : g.N / BN;
  hipLaunchKernelGGL((gemm_bf16_kernel<EPI, BM, BN>), dim3(nTM * nTN), dim3(gemm::THREADS), 0, s, g);
}

// Tile shape per launch, from the number of rounds of workgroups each shape
// needs over the 256 CUs and a per-round time relative to a round of
// 256 x 256 tiles (one per CU), measured on MI355X at K = 4096: a round of
// 128 x 256 tiles (8 waves, one per CU) takes 0.59 of it; a full round of
// 128 x 128 tiles (4 waves, two per CU) 0.65, and 0.45 when no CU gets a
// second one.  All three issue the same MFMA over the same K order for every
// output element, so the choice never changes a result bit.
enum GemmShape { SHAPE_256x256, SHAPE_128x256, SHAPE_128x128 };

// The cheapest shape for g and its cost (in hundredths of a 256 x 256 round).
template <int EPI>
GemmShape gemm_shape(const GemmArgs &g, int &grid, int &cost) {
  const int n_out = EPI == EPI_SWIGLU ? g.F : g.N;
  const int per_tile_w = EPI == EPI_SWIGLU ? 128 : 256;  // outputs of a 256-row W tile
  const int ks = g.ksplit > 1 ? g.ksplit : 1;
  const int cols_w = n_out % per_tile_w == 0 ? n_out / per_tile_w : 0;
  const int tiles_256 = ((g.M + 255) / 256) * cols_w * ks;
  const int tiles_128w = ((g.M + 127) / 128) * cols_w * ks;
  const int tiles_128 = ((g.M + 127) / 128) * (EPI == EPI_SWIGLU ? g.F / 64 : g.N / 128) * ks;
  auto rounds = [](int tiles, int per_round) { return (tiles + per_round - 1) / per_round; };
  const int c256 = cols_w ? 100 * rounds(tiles_256, 256) : INT32_MAX;
  const int c128w = cols_w ? 59 * rounds(tiles_128w, 256) : INT32_MAX;
  const int c128 = tiles_128 <= 256 ? 45 : 65 * rounds(tiles_128, 512);
  if (c256 <= c128w && c256 <= c128) {
    grid = tiles_256;
    cost = c256;
    return SHAPE_256x256;
  }
  if (c128w <= c128) {
    grid = tiles_128w;
    cost = c128w;
    return SHAPE_128x256;
  }
  grid = tiles_128;
  cost = c128;
  return SHAPE_128x128;
}

template <int EPI>
void launch_gemm_shape(const GemmArgs &g, GemmShape shape, int grid, hipStream_t s) {
  if (shape == SHAPE_256x256)
    hipLaunchKernelGGL((gemm_bf16_lds_kernel<EPI, 256, 256, 8>), dim3(grid), dim3(512), 0, s, g);
  else if (shape == SHAPE_128x256)
    hipLaunchKernelGGL((gemm_bf16_large_kernel<EPI, 2, 4, 128>), dim3(grid), dim3(gemmL::THREADS), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_bf16_mid_kernel<EPI>), dim3(grid), dim3(gemmM::THREADS), 0, s, g);
}

// The rows past the last multiple of 256 as a launch of their own: a pass
// whose row count is a little over a multiple of 256 (the joint pass at
// 1024^2: 4503 rows) would otherwise need a nearly empty extra round of
// 256-row tiles.  The tail must hold image rows only (text rows index their
// outputs from the pass's first row); its arguments see the same rows through
// offset operands and a negative text-row count, so every output element
// gets the same MFMA sequence as in one launch.
template <int EPI>
GemmArgs gemm_tail(const GemmArgs &g, int m_main) {
  GemmArgs t = g;
  t.M = g.M - m_main;
  t.A = g.A + (size_t)m_main * g.lda;
  t.L_rows = g.L_rows - m_main;
  if (EPI == EPI_F32) t.C = g.C + (size_t)m_main * g.ldc;
  if (EPI == EPI_RESID) t.X = g.X + (size_t)m_main * g.ldx;
  if (EPI == EPI_SWIGLU) t.out = g.out + (size_t)m_main * g.ldo;
  return t;
}

template <int EPI>
qi_status launch_gemm(const GemmArgs &g, int kind, hipStream_t s) {
  // the LDS-copy kernels address each operand with a 32-bit buffer offset
  const bool fits32 = (size_t)g.M * g.lda * 2 < (1ull << 31) &&
                      (size_t)(EPI == EPI_SWIGLU ? 2 * g.F : g.N) * g.ldw * 2 < (1ull << 31);
  {
    TimedLaunch tl(kind, s);
    if (!fits32) {
      const int tiles = ((g.M + 127) / 128) * (EPI == EPI_SWIGLU ? g.F / 64 : g.N / 128);
      if (EPI == EPI_RESID && g.ksplit > 1)
        hipLaunchKernelGGL((gemm_bf16_kernel<EPI, 128, 128>), dim3(tiles * g.ksplit), dim3(gemm::THREADS), 0, s, g);
      else
        launch_gemm_tile<EPI, 128, 128>(g, s);
    } else {
      int grid = 0, cost = 0;
      const GemmShape shape = gemm_shape<EPI>(g, grid, cost);
      // the cheapest split into a head of 256-row multiples (>= 2048 rows,
      // holding every text row) and an image-row tail, if any beats one launch
      bool two = false;
      GemmArgs head = g, tail{};
      int grid_h = 0, grid_t = 0;
      GemmShape shape_h = shape, shape_t = shape;
      if (g.ksplit <= 1) {
        int best = cost - 10;  // a second launch costs about a tenth of a round
        for (int m_main = g.M / 256 * 256; m_main >= 2048 && m_main >= g.L_rows; m_main -= 256) {
          if (m_main == g.M) continue;
          GemmArgs h = g;
          h.M = m_main;
          const GemmArgs t = gemm_tail<EPI>(g, m_main);
          int gh = 0, gt = 0, ch = 0, ct = 0;
          const GemmShape sh = gemm_shape<EPI>(h, gh, ch), st = gemm_shape<EPI>(t, gt, ct);
          if (ch + ct < best) {
            best = ch + ct;
            two = true;
            head = h, tail = t, grid_h = gh, grid_t = gt, shape_h = sh, shape_t = st;
          }
        }
      }
      if (two) {
        launch_gemm_shape<EPI>(head, shape_h, grid_h, s);
        launch_gemm_shape<EPI>(tail, shape_t, grid_t, s);
      } else {
        launch_gemm_shape<EPI>(g, shape, grid, s);
      }
    }
  }
  QI_TRY(last_launch());
  if (EPI == EPI_RESID && g.ksplit > 1) {
    TimedLaunch tl(QI_KERNEL_SPLITK_REDUCE, s);
    const size_t n4 = (size_t)g.M * (g.N / 4);
    hipLaunchKernelGGL(resid_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, g);
    QI_TRY(last_launch());
  }
  return QI_OK;
}

// img-in embed of N image tokens into x rows row0.. (ldx = H): four 32-token
// blocks per workgroup from N = 4096 on (a W slice loaded once serves 128
// tokens; 35 -> 24 us at N = 4096 on MI355X), one below, where four would
// leave CUs idle (N = 256: 10 -> 14 us).
void launch_img_embed(const float *img_tokens, int N, const qi_model_w &w, int H, float *x, int row0,
                      hipStream_t s) {
  if (N >= 4096)
    hipLaunchKernelGGL(img_embed_kernel<4>, dim3((N + 127) / 128, H / 256), dim3(256), 0, s, img_tokens, N, w.w_img,
                       w.b_img, H, x, H, row0);
  else
    hipLaunchKernelGGL(img_embed_kernel<1>, dim3((N + 31) / 32, H / 256), dim3(256), 0, s, img_tokens, N, w.w_img,
                       w.b_img, H, x, H, row0);
}

// The output head over `rows` rows of x [rows][H]; H % 256 == 0 (checked with
// the model dimensions).
void launch_head(const float *x, int H, int rows, const qi_model_w &w, float eps, float *vel, hipStream_t s) {
  hipLaunchKernelGGL(head_kernel<2>, dim3((rows + 15) / 16), dim3(512), 0, s, x, H, rows, w.norm_out, w.w_out, w.b_out,
                     H, eps, vel);
}

qi_status launch_norm(const float *x, int ldx, const float *gamma, int zc, const float *mod,
                      int mod_img_off, int L_rows, int rows, int H, u16 *out, int ldo, hipStream_t s,
                      const int *skip = nullptr) {
  TimedLaunch tl(zc ? QI_KERNEL_TXT_NORM : QI_KERNEL_NORM_MOD, s);
  const dim3 grid((rows + 3) / 4);
  if (H <= 4096)
    hipLaunchKernelGGL(rmsnorm_mod_kernel<16>, grid, dim3(256), 0, s, x, ldx, gamma, zc, mod, mod_img_off, L_rows,
                       rows, H, kRmsEps, out, ldo, skip);
  else
    hipLaunchKernelGGL(rmsnorm_mod_kernel<32>, grid, dim3(256), 0, s, x, ldx, gamma, zc, mod, mod_img_off, L_rows,
                       rows, H, kRmsEps, out, ldo, skip);
  return last_launch();
}

// The modulation GEMV (H % 256 == 0 and H <= 8192 are checked with the model
// dimensions): 4H rows over 256 workgroups (one per CU), at least 16 rows
// each (8 waves, one pair of rows per wave at a time).
template <int NC>
void launch_mod_gemv(int H, const u16 *w_mod, const float *b_mod, float t, float *mod, hipStream_t s) {
  const int rows = 4 * H;
  const int per = max(16, (rows + 255) / 256 + 15) & ~15;
  hipLaunchKernelGGL(mod_gemv_kernel<NC>, dim3((rows + per - 1) / per), dim3(512), 2 * H * sizeof(float), s, w_mod,
                     b_mod, t, H, rows, per, mod);
}

qi_status launch_modulation(int H, const u16 *w_mod, const float *b_mod, float t, float *mod, hipStream_t s) {
  TimedLaunch tl(QI_KERNEL_MODULATION, s);
  switch ((H + 511) / 512) {
    case 1: launch_mod_gemv<1>(H, w_mod, b_mod, t, mod, s); break;
    case 2: launch_mod_gemv<2>(H, w_mod, b_mod, t, mod, s); break;
    case 3: launch_mod_gemv<3>(H, w_mod, b_mod, t, mod, s); break;
    case 4: launch_mod_gemv<4>(H, w_mod, b_mod, t, mod, s); break;
    case 5: launch_mod_gemv<5>(H, w_mod, b_mod, t, mod, s); break;
    case 6: launch_mod_gemv<6>(H, w_mod, b_mod, t, mod, s); break;
    case 7: launch_mod_gemv<7>(H, w_mod, b_mod, t, mod, s); break;
    case 8: launch_mod_gemv<8>(H, w_mod, b_mod, t, mod, s); break;
    case 9: launch_mod_gemv<9>(H, w_mod, b_mod, t, mod, s); break;
    case 10: launch_mod_gemv<10>(H, w_mod, b_mod, t, mod, s); break;
    case 11: launch_mod_gemv<11>(H, w_mod, b_mod, t, mod, s); break;
    case 12: launch_mod_gemv<12>(H, w_mod, b_mod, t, mod, s); break;
    case 13: launch_mod_gemv<13>(H, w_mod, b_mod, t, mod, s); break;
    case 14: launch_mod_gemv<14>(H, w_mod, b_mod, t, mod, s); break;
    case 15: launch_mod_gemv<15>(H, w_mod, b_mod, t, mod, s); break;
    case 16: launch_mod_gemv<16>(H, w_mod, b_mod, t, mod, s); break;
    default: return QI_ERR_SHAPE;
  }
  return last_launch();
}

AttnArgs attn_args(int heads, int L, int N, bool joint, const u16 *q_t, const u16 *k_t, const u16 *vt_t,
                   const u16 *q_i, const u16 *k_i, const u16 *vt_i, u16 *o) {
  AttnArgs a{};
  a.q_t = q_t; a.k_t = k_t; a.vt_t = vt_t;
  a.q_i = q_i; a.k_i = k_i; a.vt_i = vt_i;
  a.o = o;
  a.ldo = heads * 128;
  a.heads = heads; a.L = L; a.N = N;
  a.ldv_t = round64(L); a.ldv_i = round64(N);
  a.joint = joint ? 1 : 0;
  a.o_img_row0 = joint ? L : 0;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt(128.0));
  return a;
}

qi_status launch_attention_batch(const AttnBatch &ab, hipStream_t s) {
  TimedLaunch tl(QI_KERNEL_ATTENTION, s);
  launch_block_causal_attn(ab, s);
  return last_launch();
}

qi_status launch_attention(int heads, int L, int N, bool joint, const u16 *q_t, const u16 *k_t,
                           const u16 *vt_t, const u16 *q_i, const u16 *k_i, const u16 *vt_i, u16 *o,
                           hipStream_t s, const int *skip = nullptr) {
  AttnBatch ab{};
  ab.br[0] = attn_args(heads, L, N, joint, q_t, k_t, vt_t, q_i, k_i, vt_i, o);
  ab.br[0].skip = skip;
  ab.nbranch = 1;
  return launch_attention_batch(ab, s);
}

// The launch sequence of one block; arguments already validated.
//
// Two-branch form (true CFG, image-only): nb = 2, rows [branch 0 | branch 1]
// of N image rows each, cos_i/sin_i holding 2N rows, branch b reading its text
// K/V from kv_slot (b = 0, L rows) or kv_slot2 (b = 1, L2 rows).  Every GEMM,
// norm and the attention run once over both branches; each row's result is
// the one the single-branch pass computes (row-count invariance).
qi_status run_block(const qi_dims &d, const qi_block_w &w, int L, int N, bool joint, float *x,
                    const float *mod, const float *cos_t, const float *sin_t, const float *cos_i,
                    const float *sin_i, u16 *kv_slot, char *ws, const Layout &lay, hipStream_t s,
                    int nb = 1, u16 *kv_slot2 = nullptr, int L2 = 0, const int *skip = nullptr) {
  const int H = d.hidden, F = d.ffn, heads = d.heads;
  const int L_rows = joint ? L : 0, T = L_rows + nb * N;
  const int img_off = 4 * H;  // mod row 1
  u16 *h = (u16 *)(ws + lay.h);
  u16 *o = (u16 *)(ws + lay.o);
  u16 *a = (u16 *)(ws + lay.a);
  u16 *q_t = (u16 *)(ws + lay.q_t);
  u16 *k_t = kv_slot ? kv_slot : (u16 *)(ws + lay.k_t);
  u16 *vt_t = kv_slot ? kv_slot + (size_t)heads * L * 128 : (u16 *)(ws + lay.vt_t);
  u16 *q_i = (u16 *)(ws + lay.q_i), *k_i = (u16 *)(ws + lay.k_i), *vt_i = (u16 *)(ws + lay.vt_i);

  // norm 1 + modulation (scale1 = chunk 0)
  QI_TRY(launch_norm(x, H, w.norm1, 0, mod, img_off, L_rows, T, H, h, H, s, skip));

  // QKV + RoPE (+ text K/V into the cache slot on a capture pass)
  GemmArgs g{};
  g.A = h; g.lda = H; g.W = w.w_qkv; g.ldw = H; g.M = T; g.N = 3 * H; g.K = H; g.L_rows = L_rows;
  g.H = H;
  g.cos_t = cos_t; g.sin_t = sin_t; g.cos_i = cos_i; g.sin_i = sin_i;
  g.q_t = q_t; g.k_t = k_t; g.vt_t = vt_t; g.q_i = q_i; g.k_i = k_i; g.vt_i = vt_i;
  g.seg_t = L; g.seg_i = N; g.ldv_t = round64(L); g.ldv_i = round64(N);
  g.batch = nb;
  g.skip = skip;
  QI_TRY(launch_gemm<EPI_QKV>(g, QI_KERNEL_GEMM_QKV, s));

  if (nb == 1) {
    QI_TRY(launch_attention(heads, L, N, joint, q_t, k_t, vt_t, q_i, k_i, vt_i, o, s, skip));
  } else {
    AttnBatch ab{};
    ab.nbranch = 2;
    ab.br[0] = attn_args(heads, L, N, false, nullptr, k_t, vt_t, q_i, k_i, vt_i, o);
    ab.br[1] = attn_args(heads, L2, N, false, nullptr, kv_slot2, kv_slot2 + (size_t)heads * L2 * 128,
                         q_i + (size_t)H * N, k_i + (size_t)H * N, vt_i + (size_t)H * round64(N),
                         o + (size_t)N * H);
    ab.br[0].skip = ab.br[1].skip = skip;
    QI_TRY(launch_attention_batch(ab, s));
  }

  // O projection + gated residual 1 (gate1 = chunk 1)
  GemmArgs r{};
  r.A = o; r.lda = H; r.W = w.w_o; r.ldw = H; r.M = T; r.N = H; r.K = H; r.L_rows = L_rows;
  r.X = x; r.ldx = H; r.gate = mod + H; r.gate_img_off = img_off;
  r.skip = skip;
  r.ksplit = ksplit_o(d, N);
  r.part = (float *)(ws + lay.part);
  QI_TRY(launch_gemm<EPI_RESID>(r, QI_KERNEL_GEMM_O, s));

  // norm 2 + modulation (scale2 = chunk 2)
  QI_TRY(launch_norm(x, H, w.norm2, 0, mod + 2 * H, img_off, L_rows, T, H, h, H, s, skip));

  // gate/up + SwiGLU
  GemmArgs u{};
  u.A = h; u.lda = H; u.W = w.w_gu; u.ldw = H; u.M = T; u.N = 2 * F; u.K = H; u.L_rows = L_rows;
  u.out = a; u.ldo = F; u.F = F;
  u.skip = skip;
  QI_TRY(launch_gemm<EPI_SWIGLU>(u, QI_KERNEL_GEMM_GATE_UP, s));

  // down + gated residual 2 (gate2 = chunk 3)
  GemmArgs dn{};
  dn.A = a; dn.lda = F; dn.W = w.w_down; dn.ldw = F; dn.M = T; dn.N = H; dn.K = F; dn.L_rows = L_rows;
  dn.X = x; dn.ldx = H; dn.gate = mod + 3 * H; dn.gate_img_off = img_off;
  dn.skip = skip;
  dn.ksplit = ksplit_down(d, N);
  dn.part = (float *)(ws + lay.part);
  QI_TRY(launch_gemm<EPI_RESID>(dn, QI_KERNEL_GEMM_DOWN, s));
  return QI_OK;
}

qi_status check_block_w(const qi_block_w *w) {
  if (!w || !w->w_qkv || !w->w_o || !w->w_gu || !w->w_down || !w->norm1 || !w->norm2) return QI_ERR_NULL;
  if (!al16(w->w_qkv) || !al16(w->w_o) || !al16(w->w_gu) || !al16(w->w_down) || !al16(w->norm1) ||
      !al16(w->norm2))
    return QI_ERR_ALIGN;
  return QI_OK;
}

qi_status check_model_w(const qi_dims &d, const qi_model_w *w, bool need_text) {
  if (!w || !w->blocks || !w->w_mod || !w->b_mod || !w->w_img || !w->b_img || !w->norm_out || !w->w_out ||
      !w->b_out)
    return QI_ERR_NULL;
  if (need_text && (!w->txt_norm || !w->w_txt || !w->b_txt)) return QI_ERR_NULL;
  const void *ps[] = {w->w_mod, w->b_mod, w->w_img, w->b_img, w->norm_out, w->w_out, w->b_out};
  for (const void *p : ps)
    if (!al16(p)) return QI_ERR_ALIGN;
  if (need_text && (!al16(w->txt_norm) || !al16(w->w_txt) || !al16(w->b_txt))) return QI_ERR_ALIGN;
  for (int b = 0; b < d.n_blocks; ++b) QI_TRY(check_block_w(&w->blocks[b]));
  return QI_OK;
}

// A whole step: joint when kv == NULL or capture, image-only otherwise.
qi_status run_step(const qi_dims &d, const qi_model_w &w, int L, int N, const float *img_tokens,
                   const float *txt_feats, float t, const float *txt_cos, const float *txt_sin,
                   const float *img_cos, const float *img_sin, u16 *kv, bool joint, float *vel,
                   char *ws, hipStream_t s) {
  const int H = d.hidden, D = d.txt_dim;
  const Layout lay = layout(d, L, N);
  float *x = (float *)(ws + lay.x);
  float *mod = (float *)(ws + lay.mod);
  const int L_rows = joint ? L : 0;

  QI_TRY(launch_modulation(H, w.w_mod, w.b_mod, t, mod, s));

  if (joint) {
    u16 *tn = (u16 *)(ws + lay.tn);
    QI_TRY(launch_norm(txt_feats, D, w.txt_norm, 1, nullptr, 0, 0, L, D, tn, D, s));
    GemmArgs g{};
    g.A = tn; g.lda = D; g.W = w.w_txt; g.ldw = D; g.M = L; g.N = H; g.K = D; g.L_rows = L;
    g.C = x; g.ldc = H; g.bias = w.b_txt;
    QI_TRY(launch_gemm<EPI_F32>(g, QI_KERNEL_GEMM_TXT, s));
  }
  {
    TimedLaunch tl(QI_KERNEL_IMG_EMBED, s);
    launch_img_embed(img_tokens, N, w, H, x, L_rows, s);
  }
  QI_TRY(last_launch());

  const size_t slot = slot_elems(d, L);
  for (int b = 0; b < d.n_blocks; ++b) {
    u16 *kv_slot = kv ? kv + (size_t)b * slot : nullptr;
    QI_TRY(run_block(d, w.blocks[b], L, N, joint, x, mod, txt_cos, txt_sin, img_cos, img_sin, kv_slot, ws,
                     lay, s));
  }
  if (vel) {
    TimedLaunch tl(QI_KERNEL_HEAD, s);
    launch_head(x + (size_t)L_rows * H, H, N, w, kRmsEps, vel, s);
    QI_TRY(last_launch());
  }
  return QI_OK;
}

// ---------------------------------------------------------------- text encoder
bool enc_dims_ok(const qi_enc_dims *d) {
  if (!d) return false;
  if (d->head_dim != 128 || d->heads < 1 || d->kv_heads < 1 || d->heads % d->kv_heads != 0) return false;
  if (d->hidden < 256 || d->hidden > 16384 || d->hidden % 256 != 0) return false;
  if (d->ffn < 64 || d->ffn % 64 != 0 || d->ffn > 65536) return false;
  if (d->n_layers < 1 || d->n_layers > 256 || d->vocab < 1) return false;
  if ((size_t)d->heads * 128 > 65536) return false;
  // every weight matrix addressed with 32-bit byte offsets
  const size_t H = d->hidden, F = d->ffn, NQ = (size_t)d->heads * 128, NT = NQ + (size_t)2 * d->kv_heads * 128;
  if (NT * H * 2 >= (1ull << 31) || H * NQ * 2 >= (1ull << 31) || 2 * F * H * 2 >= (1ull << 31) ||
      H * F * 2 >= (1ull << 31))
    return false;
  return true;
}

struct EncLayout {
  size_t h, qkv, q, k, v, o, a, total;
};
EncLayout enc_layout(const qi_enc_dims &d, int L) {
  const size_t H = d.hidden, NQ = (size_t)d.heads * 128, NKV = (size_t)d.kv_heads * 128, F = d.ffn;
  EncLayout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  l.h = take((size_t)3 * L * H * 2);  // bf16 planes of the normed rows
  l.qkv = take((size_t)L * (NQ + 2 * NKV) * 4);
  l.q = take((size_t)L * NQ * 4);
  l.k = take((size_t)L * NKV * 4);
  l.v = take((size_t)L * NKV * 4);
  l.o = take((size_t)3 * L * NQ * 2);  // planes of the attention output
  l.a = take((size_t)3 * L * F * 2);   // planes of the SwiGLU output
  l.total = off;
  return l;
}

template <int EPI>
qi_status launch_enc_gemm(const EncGemmArgs &g, hipStream_t s) {
  const int nTM = (g.M + enc::BM - 1) / enc::BM;
  const int nTN = EPI == ENC_SWIGLU ? g.F / (enc::BN / 2) : g.N / enc::BN;
  TimedLaunch tl(QI_KERNEL_ENC_GEMM, s);
  hipLaunchKernelGGL((enc_gemm_kernel<EPI>), dim3(nTM * nTN), dim3(enc::THREADS), 0, s, g);
  return last_launch();
}

// The encoder forward; arguments validated.  x is the caller's hidden buffer.
qi_status run_encoder(const qi_enc_dims &d, const qi_enc_model_w &w, const int32_t *ids, int L, const float *cos,
                      const float *sin, float *x, char *ws, hipStream_t s) {
  const int H = d.hidden, F = d.ffn, NQ = d.heads * 128, NKV = d.kv_heads * 128, NT = NQ + 2 * NKV;
  const EncLayout lay = enc_layout(d, L);
  u16 *h = (u16 *)(ws + lay.h), *O = (u16 *)(ws + lay.o), *a = (u16 *)(ws + lay.a);
  float *qkv = (float *)(ws + lay.qkv), *Q = (float *)(ws + lay.q), *K = (float *)(ws + lay.k),
        *V = (float *)(ws + lay.v);
  {
    TimedLaunch tl(QI_KERNEL_ENC_MISC, s);
    hipLaunchKernelGGL(enc_embed_kernel, dim3(L), dim3(256), 0, s, ids, d.vocab, w.embed, H, x);
  }
  QI_TRY(last_launch());
  for (int li = 0; li < d.n_layers; ++li) {
    const qi_enc_layer_w &lw = w.layers[li];
    {
      TimedLaunch tl(QI_KERNEL_ENC_MISC, s);
      hipLaunchKernelGGL(enc_rmsnorm_kernel, dim3((L + 3) / 4), dim3(256), 0, s, x, lw.in_norm, L, H, kRmsEps, h);
    }
    QI_TRY(last_launch());
    EncGemmArgs g{};
    g.A = h; g.lda = H; g.W = lw.w_qkv; g.ldw = H; g.M = L; g.N = NT; g.K = H; g.C = qkv; g.ldc = NT;
    QI_TRY(launch_enc_gemm<ENC_F32>(g, s));
    {
      TimedLaunch tl(QI_KERNEL_ENC_MISC, s);
      const int waves = L * (d.heads + 2 * d.kv_heads);
      hipLaunchKernelGGL(enc_qk_prep_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, qkv, L, d.heads, d.kv_heads,
                         lw.q_norm, lw.k_norm, cos, sin, kRmsEps, Q, K, V);
    }
    QI_TRY(last_launch());
    {
      TimedLaunch tl(QI_KERNEL_ENC_ATTN, s);
      hipLaunchKernelGGL(enc_attention_kernel, dim3((L + enca::BQ - 1) / enca::BQ, d.heads), dim3(256), 0, s, Q,
                         K, V, O, L, d.heads, d.kv_heads);
    }
    QI_TRY(last_launch());
    EncGemmArgs r{};
    r.A = O; r.lda = NQ; r.W = lw.w_o; r.ldw = NQ; r.M = L; r.N = H; r.K = NQ; r.X = x; r.ldx = H;
    QI_TRY(launch_enc_gemm<ENC_RESID>(r, s));
    {
      TimedLaunch tl(QI_KERNEL_ENC_MISC, s);
      hipLaunchKernelGGL(enc_rmsnorm_kernel, dim3((L + 3) / 4), dim3(256), 0, s, x, lw.post_norm, L, H, kRmsEps,
                         h);
    }
    QI_TRY(last_launch());
    EncGemmArgs u{};
    u.A = h; u.lda = H; u.W = lw.w_gu; u.ldw = H; u.M = L; u.N = 2 * F; u.K = H; u.out = a; u.ldo = F; u.F = F;
    QI_TRY(launch_enc_gemm<ENC_SWIGLU>(u, s));
    EncGemmArgs dn{};
    dn.A = a; dn.lda = F; dn.W = lw.w_down; dn.ldw = F; dn.M = L; dn.N = H; dn.K = F; dn.X = x; dn.ldx = H;
    QI_TRY(launch_enc_gemm<ENC_RESID>(dn, s));
  }
  return QI_OK;
}

// First-block-cache buffer: state, partial sums, then x0, r0p (cached block-0
// residual), x1s (x after block 0 on the last computed step) and rem (cached
// residual of blocks 1..n-1), each [N][H] fp32.
constexpr int kFbcParts = 512;
struct FbcLayout {
  size_t state, part, x0, r0p, x1s, rem, total;
};
FbcLayout fbc_layout(const qi_dims &d, int N) {
  const size_t X = (size_t)N * d.hidden * 4;
  FbcLayout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  l.state = take(sizeof(FbcState));
  l.part = take(2 * kFbcParts * sizeof(double));
  l.x0 = take(X);
  l.r0p = take(X);
  l.x1s = take(X);
  l.rem = take(X);
  l.total = off;
  return l;
}

// An image-only step with the first-block cache ([MLX] "Optional modes", Fast
// mode): block 0, the on-device decision, then blocks 1..n-1 whose kernels all
// return at once when the step is skipped.  No host synchronisation.
qi_status run_step_fbc(const qi_dims &d, const qi_model_w &w, int L, int N, const float *img_tokens, float t,
                       const float *img_cos, const float *img_sin, u16 *kv, float threshold, char *fbc,
                       float *vel, char *ws, hipStream_t s) {
  const int H = d.hidden;
  const Layout lay = layout(d, L, N);
  const FbcLayout fl = fbc_layout(d, N);
  float *x = (float *)(ws + lay.x);
  float *mod = (float *)(ws + lay.mod);
  FbcState *st = (FbcState *)(fbc + fl.state);
  double *part = (double *)(fbc + fl.part);
  float *x0 = (float *)(fbc + fl.x0), *r0p = (float *)(fbc + fl.r0p), *x1s = (float *)(fbc + fl.x1s),
        *rem = (float *)(fbc + fl.rem);
  const int64_t n4 = (int64_t)N * H / 4;
  const int eblocks = (int)((n4 + 255) / 256 < 2048 ? (n4 + 255) / 256 : 2048);
  const int pblocks = (int)((n4 + 255) / 256 < kFbcParts ? (n4 + 255) / 256 : kFbcParts);

  QI_TRY(launch_modulation(H, w.w_mod, w.b_mod, t, mod, s));
  {
    TimedLaunch tl(QI_KERNEL_IMG_EMBED, s);
    launch_img_embed(img_tokens, N, w, H, x, 0, s);
  }
  QI_TRY(last_launch());
  hipLaunchKernelGGL(fbc_copy_kernel, dim3(eblocks), dim3(256), 0, s, x0, x, n4);
  QI_TRY(last_launch());
  const size_t slot = slot_elems(d, L);
  QI_TRY(run_block(d, w.blocks[0], L, N, false, x, mod, nullptr, nullptr, img_cos, img_sin, kv, ws, lay, s));
  hipLaunchKernelGGL(fbc_partial_kernel, dim3(pblocks), dim3(256), 0, s, x, x0, r0p, n4, part);
  QI_TRY(last_launch());
  hipLaunchKernelGGL(fbc_decide_kernel, dim3(1), dim3(64), 0, s, part, pblocks, threshold, st);
  QI_TRY(last_launch());
  hipLaunchKernelGGL(fbc_apply_kernel, dim3(eblocks), dim3(256), 0, s, x, x0, r0p, x1s, rem, n4, st);
  QI_TRY(last_launch());
  for (int b = 1; b < d.n_blocks; ++b)
    QI_TRY(run_block(d, w.blocks[b], L, N, false, x, mod, nullptr, nullptr, img_cos, img_sin,
                     kv + (size_t)b * slot, ws, lay, s, 1, nullptr, 0, &st->skip));
  hipLaunchKernelGGL(fbc_finish_kernel, dim3(eblocks), dim3(256), 0, s, x, x1s, rem, n4, st);
  QI_TRY(last_launch());
  TimedLaunch tl(QI_KERNEL_HEAD, s);
  launch_head(x, H, N, w, kRmsEps, vel, s);
  return last_launch();
}

// A true-CFG image-only step: both branches through every block at once,
// vel = [pos | neg] ([2N, 64]).
qi_status run_step_cfg(const qi_dims &d, const qi_model_w &w, int N, const float *img_tokens, float t,
                       const float *img_cos, const float *img_sin, u16 *kv_pos, int L_pos, u16 *kv_neg,
                       int L_neg, float *vel, char *ws, hipStream_t s) {
  const int H = d.hidden;
  const Layout lay = layout_cfg(d, N);
  float *x = (float *)(ws + lay.x);
  float *mod = (float *)(ws + lay.mod);
  QI_TRY(launch_modulation(H, w.w_mod, w.b_mod, t, mod, s));
  for (int b = 0; b < 2; ++b) {
    TimedLaunch tl(QI_KERNEL_IMG_EMBED, s);
    launch_img_embed(img_tokens, N, w, H, x, b * N, s);
    QI_TRY(last_launch());
  }
  const size_t slot_p = slot_elems(d, L_pos), slot_n = slot_elems(d, L_neg);
  for (int b = 0; b < d.n_blocks; ++b)
    QI_TRY(run_block(d, w.blocks[b], L_pos, N, false, x, mod, nullptr, nullptr, img_cos, img_sin,
                     kv_pos + (size_t)b * slot_p, ws, lay, s, 2, kv_neg + (size_t)b * slot_n, L_neg));
  TimedLaunch tl(QI_KERNEL_HEAD, s);
  launch_head(x, H, 2 * N, w, kRmsEps, vel, s);
  return last_launch();
}

qi_status check_step_args(const qi_dims *d, const qi_model_w *w, int L, int N, const float *img_tokens,
                          const float *txt_feats, float t, const float *txt_cos, const float *txt_sin,
                          const float *img_cos, const float *img_sin, bool joint, const void *ws,
                          size_t ws_bytes) {
  if (!d) return QI_ERR_NULL;
  if (!dims_ok(d)) return QI_ERR_SHAPE;
  if (L < 1 || L > kMaxL || N < 1 || N > kMaxN) return QI_ERR_RANGE;
  if (!(t >= 0.f && t <= 1.f)) return QI_ERR_RANGE;
  if (!img_tokens || !img_cos || !img_sin || !ws) return QI_ERR_NULL;
  if (joint && (!txt_feats || !txt_cos || !txt_sin)) return QI_ERR_NULL;
  if (!al16(img_tokens) || !al16(img_cos) || !al16(img_sin) || !al16(ws)) return QI_ERR_ALIGN;
  if (joint && (!al16(txt_feats) || !al16(txt_cos) || !al16(txt_sin))) return QI_ERR_ALIGN;
  QI_TRY(check_model_w(*d, w, joint));
  if (ws_bytes < layout(*d, L, N).total) return QI_ERR_WORKSPACE;
  return QI_OK;
}

}  // namespace

extern "C" {

const char *qi_status_str(qi_status s) {
  switch (s) {
    case QI_OK: return "ok";
    case QI_ERR_NULL: return "a required pointer is NULL";
    case QI_ERR_SHAPE: return "inconsistent dimensions";
    case QI_ERR_RANGE: return "a size is outside its supported range";
    case QI_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case QI_ERR_WORKSPACE: return "workspace smaller than qi_workspace_bytes";
    case QI_ERR_CACHE: return "K/V cache invalid or made for another shape";
    case QI_ERR_HIP: return "a HIP call or kernel launch failed";
    case QI_ERR_UNSUPPORTED: return "unsupported request";
    default: return "unknown status";
  }
}

const char *qi_version(void) { return "qi-dit-gfx950 0.1"; }

size_t qi_workspace_bytes(const qi_dims *d, int32_t L, int32_t N) {
  if (!dims_ok(d) || L < 1 || L > kMaxL || N < 1 || N > kMaxN) return 0;
  return layout(*d, L, N).total;
}

size_t qi_kv_slot_elems(const qi_dims *d, int32_t L) {
  if (!dims_ok(d) || L < 1 || L > kMaxL) return 0;
  return slot_elems(*d, L);
}

size_t qi_kv_cache_bytes(const qi_dims *d, int32_t L) {
  if (!dims_ok(d) || L < 1 || L > kMaxL) return 0;
  return slot_elems(*d, L) * 2 * (size_t)d->n_blocks;
}

qi_status qi_dit_block_fwd(const qi_dims *d, const qi_block_w *w, int32_t L, int32_t N, int32_t mode,
                           float *x, const float *mod, const float *cos, const float *sin, uint16_t *kv_txt,
                           void *ws, size_t ws_bytes, void *stream) {
  if (!d) return QI_ERR_NULL;
  if (!dims_ok(d)) return QI_ERR_SHAPE;
  if (mode != QI_MODE_JOINT && mode != QI_MODE_IMAGE_ONLY) return QI_ERR_RANGE;
  if (L < 1 || L > kMaxL || N < 1 || N > kMaxN) return QI_ERR_RANGE;
  if (!x || !mod || !cos || !sin || !ws) return QI_ERR_NULL;
  const bool joint = mode == QI_MODE_JOINT;
  if (!joint && !kv_txt) return QI_ERR_CACHE;
  if (!al16(x) || !al16(mod) || !al16(cos) || !al16(sin) || !al16(ws) || (kv_txt && !al16(kv_txt)))
    return QI_ERR_ALIGN;
  QI_TRY(check_block_w(w));
  const Layout lay = layout(*d, L, N);
  if (ws_bytes < lay.total) return QI_ERR_WORKSPACE;
  const int L_rows = joint ? L : 0;
  const float *cos_t = cos, *sin_t = sin;
  const float *cos_i = cos + (size_t)L_rows * 64, *sin_i = sin + (size_t)L_rows * 64;
  return run_block(*d, *w, L, N, joint, x, mod, cos_t, sin_t, cos_i, sin_i, kv_txt, (char *)ws, lay,
                   (hipStream_t)stream);
}

qi_status qi_dit_step(const qi_dims *d, const qi_model_w *w, int32_t L, int32_t N, const float *img_tokens,
                      const float *txt_feats, float timestep, const float *txt_cos, const float *txt_sin,
                      const float *img_cos, const float *img_sin, const qi_kv_cache *cache, float *vel,
                      void *ws, size_t ws_bytes, void *stream) {
  const bool joint = cache == nullptr;
  QI_TRY(check_step_args(d, w, L, N, img_tokens, txt_feats, timestep, txt_cos, txt_sin, img_cos, img_sin,
                         joint, ws, ws_bytes));
  if (!vel) return QI_ERR_NULL;
  if (!al16(vel)) return QI_ERR_ALIGN;
  if (cache) {
    if (!cache->kv || !cache->valid || cache->L != L || cache->n_blocks != d->n_blocks ||
        cache->hidden != d->hidden)
      return QI_ERR_CACHE;
    if (!al16(cache->kv)) return QI_ERR_ALIGN;
  }
  return run_step(*d, *w, L, N, img_tokens, txt_feats, timestep, txt_cos, txt_sin, img_cos, img_sin,
                  cache ? cache->kv : nullptr, joint, vel, (char *)ws, (hipStream_t)stream);
}

qi_status qi_text_kv_capture(const qi_dims *d, const qi_model_w *w, int32_t L, int32_t N,
                             const float *img_tokens, const float *txt_feats, float timestep,
                             const float *txt_cos, const float *txt_sin, const float *img_cos,
                             const float *img_sin, qi_kv_cache *cache, float *vel, void *ws, size_t ws_bytes,
                             void *stream) {
  QI_TRY(check_step_args(d, w, L, N, img_tokens, txt_feats, timestep, txt_cos, txt_sin, img_cos, img_sin,
                         true, ws, ws_bytes));
  if (!cache || !cache->kv) return QI_ERR_NULL;
  if (!al16(cache->kv) || (vel && !al16(vel))) return QI_ERR_ALIGN;
  cache->valid = 0;
  QI_TRY(run_step(*d, *w, L, N, img_tokens, txt_feats, timestep, txt_cos, txt_sin, img_cos, img_sin, cache->kv,
                  true, vel, (char *)ws, (hipStream_t)stream));
  cache->L = L;
  cache->n_blocks = d->n_blocks;
  cache->hidden = d->hidden;
  cache->valid = 1;
  return QI_OK;
}

size_t qi_cfg_workspace_bytes(const qi_dims *d, int32_t N) {
  if (!d || !dims_ok(d) || N < 1 || N > kMaxN) return 0;
  return layout_cfg(*d, N).total;
}

qi_status qi_dit_step_cfg(const qi_dims *d, const qi_model_w *w, int32_t N, const float *img_tokens,
                          float timestep, const float *img_cos, const float *img_sin, const qi_kv_cache *cache_pos,
                          const qi_kv_cache *cache_neg, float *vel, void *ws, size_t ws_bytes, void *stream) {
  if (!d) return QI_ERR_NULL;
  if (!dims_ok(d)) return QI_ERR_SHAPE;
  if (N < 1 || N > kMaxN) return QI_ERR_RANGE;
  if (!(timestep >= 0.f && timestep <= 1.f)) return QI_ERR_RANGE;
  if (!img_tokens || !img_cos || !img_sin || !vel || !ws || !cache_pos || !cache_neg) return QI_ERR_NULL;
  if (!al16(img_tokens) || !al16(img_cos) || !al16(img_sin) || !al16(vel) || !al16(ws)) return QI_ERR_ALIGN;
  QI_TRY(check_model_w(*d, w, false));
  for (const qi_kv_cache *c : {cache_pos, cache_neg}) {
    if (!c->kv || !c->valid || c->L < 1 || c->L > kMaxL || c->n_blocks != d->n_blocks || c->hidden != d->hidden)
      return QI_ERR_CACHE;
    if (!al16(c->kv)) return QI_ERR_ALIGN;
  }
  if (cache_pos->kv == cache_neg->kv) return QI_ERR_CACHE;
  if (ws_bytes < layout_cfg(*d, N).total) return QI_ERR_WORKSPACE;
  return run_step_cfg(*d, *w, N, img_tokens, timestep, img_cos, img_sin, cache_pos->kv, cache_pos->L,
                      cache_neg->kv, cache_neg->L, vel, (char *)ws, (hipStream_t)stream);
}

qi_status qi_euler_update_cfg(float *x, const float *vel, float guidance, float sigma_cur, float sigma_next,
                              int64_t n, void *stream) {
  if (n < 0) return QI_ERR_RANGE;
  if (n == 0) return QI_OK;
  if (!x || !vel) return QI_ERR_NULL;
  if (!al16(x) || !al16(vel)) return QI_ERR_ALIGN;
  if (!std::isfinite(guidance)) return QI_ERR_RANGE;
  const float ds = sigma_next - sigma_cur;  // fp32 difference on the host
  const int64_t n4 = (n + 3) / 4;
  const int blocks = (int)((n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096);
  TimedLaunch tl(QI_KERNEL_EULER, (hipStream_t)stream);
  hipLaunchKernelGGL(euler_cfg_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, x, vel, guidance, ds, n);
  return last_launch();
}

qi_status qi_dpmpp_2m_update(float *x, const float *vel, float *x0_prev, int32_t has_prev, float sigma_prev,
                             float sigma_cur, float sigma_next, int64_t n, void *stream) {
  if (n < 0) return QI_ERR_RANGE;
  if (!x || !vel || !x0_prev) return QI_ERR_NULL;
  double c[4];
  const qi_status order = qi_dpmpp_2m_coeffs(has_prev, sigma_prev, sigma_cur, sigma_next, c);
  if (order < 0) return order;
  if (n == 0) return QI_OK;
  const int64_t blocks64 = (n + 255) / 256;
  const int blocks = (int)(blocks64 < 4096 ? blocks64 : 4096);
  TimedLaunch tl(QI_KERNEL_EULER, (hipStream_t)stream);
  hipLaunchKernelGGL(dpmpp_2m_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, x, vel, x0_prev, sigma_cur,
                     (float)c[0], (float)c[1], (float)c[2], (float)c[3], (int)order, n);
  return last_launch();
}

size_t qi_enc_workspace_bytes(const qi_enc_dims *d, int32_t L) {
  if (!enc_dims_ok(d) || L < 1 || L > kMaxL) return 0;
  return enc_layout(*d, L).total;
}

qi_status qi_text_encoder_fwd(const qi_enc_dims *d, const qi_enc_model_w *w, const int32_t *ids, int32_t L,
                              const float *cos, const float *sin, float *hidden, void *ws, size_t ws_bytes,
                              void *stream) {
  if (!d || !w) return QI_ERR_NULL;
  if (!enc_dims_ok(d)) return QI_ERR_SHAPE;
  if (L < 1 || L > kMaxL) return QI_ERR_RANGE;
  if (!ids || !cos || !sin || !hidden || !ws || !w->layers || !w->embed) return QI_ERR_NULL;
  if (!al16(cos) || !al16(sin) || !al16(hidden) || !al16(ws) || !al16(w->embed)) return QI_ERR_ALIGN;
  for (int i = 0; i < d->n_layers; ++i) {
    const qi_enc_layer_w &lw = w->layers[i];
    const void *ps[] = {lw.w_qkv, lw.q_norm, lw.k_norm, lw.w_o, lw.w_gu, lw.w_down, lw.in_norm, lw.post_norm};
    for (const void *p : ps) {
      if (!p) return QI_ERR_NULL;
      if (!al16(p)) return QI_ERR_ALIGN;
    }
  }
  if (ws_bytes < enc_layout(*d, L).total) return QI_ERR_WORKSPACE;
  return run_encoder(*d, *w, ids, L, cos, sin, hidden, (char *)ws, (hipStream_t)stream);
}

size_t qi_fbc_bytes(const qi_dims *d, int32_t N) {
  if (!d || !dims_ok(d) || N < 1 || N > kMaxN) return 0;
  return fbc_layout(*d, N).total;
}

qi_status qi_fbc_reset(void *fbc, size_t fbc_bytes, void *stream) {
  if (!fbc) return QI_ERR_NULL;
  if (!al16(fbc)) return QI_ERR_ALIGN;
  if (fbc_bytes < sizeof(FbcState)) return QI_ERR_WORKSPACE;
  hipLaunchKernelGGL(fbc_reset_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, (FbcState *)fbc);
  return last_launch();
}

qi_status qi_fbc_stats(const void *fbc, int32_t *n_steps, int32_t *n_skipped, float *last_change, void *stream) {
  if (!fbc || !n_steps || !n_skipped || !last_change) return QI_ERR_NULL;
  if (!al16(fbc)) return QI_ERR_ALIGN;
  FbcState h{};
  if (hipMemcpyAsync(&h, fbc, sizeof(h), hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess ||
      hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
    return QI_ERR_HIP;
  *n_steps = h.n_steps;
  *n_skipped = h.n_skipped;
  *last_change = h.last_change;
  return QI_OK;
}

qi_status qi_dit_step_fbc(const qi_dims *d, const qi_model_w *w, int32_t L, int32_t N, const float *img_tokens,
                          float timestep, const float *img_cos, const float *img_sin, const qi_kv_cache *cache,
                          float threshold, void *fbc, size_t fbc_bytes, float *vel, void *ws, size_t ws_bytes,
                          void *stream) {
  QI_TRY(check_step_args(d, w, L, N, img_tokens, nullptr, timestep, nullptr, nullptr, img_cos, img_sin, false, ws,
                         ws_bytes));
  if (!vel || !fbc || !cache) return QI_ERR_NULL;
  if (!al16(vel) || !al16(fbc)) return QI_ERR_ALIGN;
  if (!(threshold >= 0.f) || !std::isfinite(threshold)) return QI_ERR_RANGE;
  if (fbc_bytes < fbc_layout(*d, N).total) return QI_ERR_WORKSPACE;
  if (!cache->kv || !cache->valid || cache->L != L || cache->n_blocks != d->n_blocks || cache->hidden != d->hidden)
    return QI_ERR_CACHE;
  if (!al16(cache->kv)) return QI_ERR_ALIGN;
  return run_step_fbc(*d, *w, L, N, img_tokens, timestep, img_cos, img_sin, cache->kv, threshold, (char *)fbc, vel,
                      (char *)ws, (hipStream_t)stream);
}

qi_status qi_euler_update(float *x, const float *vel, float sigma_cur, float sigma_next, int64_t n,
                          void *stream) {
  if (n < 0) return QI_ERR_RANGE;
  if (n == 0) return QI_OK;
  if (!x || !vel) return QI_ERR_NULL;
  if (!al16(x) || !al16(vel)) return QI_ERR_ALIGN;
  const float ds = sigma_next - sigma_cur;  // fp32 difference on the host
  const int64_t n4 = (n + 3) / 4;
  const int blocks = (int)((n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096);
  TimedLaunch tl(QI_KERNEL_EULER, (hipStream_t)stream);
  hipLaunchKernelGGL(euler_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, x, vel, ds, n);
  return last_launch();
}

qi_status qi_modulation(const qi_dims *d, const uint16_t *w_mod, const float *b_mod, float timestep, float *mod,
                        void *stream) {
  if (!d) return QI_ERR_NULL;
  if (!dims_ok(d)) return QI_ERR_SHAPE;
  if (!(timestep >= 0.f && timestep <= 1.f)) return QI_ERR_RANGE;
  if (!w_mod || !b_mod || !mod) return QI_ERR_NULL;
  if (!al16(w_mod) || !al16(b_mod) || !al16(mod)) return QI_ERR_ALIGN;
  return launch_modulation(d->hidden, w_mod, b_mod, timestep, mod, (hipStream_t)stream);
}

qi_status qi_block_causal_attention(int32_t heads, int32_t L, int32_t N, int32_t mode, const uint16_t *q_txt,
                                    const uint16_t *k_txt, const uint16_t *vt_txt, const uint16_t *q_img,
                                    const uint16_t *k_img, const uint16_t *vt_img, uint16_t *o, void *stream) {
  if (heads < 1 || heads > 64 || L < 1 || L > kMaxL || N < 1 || N > kMaxN) return QI_ERR_RANGE;
  if (mode != QI_MODE_JOINT && mode != QI_MODE_IMAGE_ONLY) return QI_ERR_RANGE;
  const bool joint = mode == QI_MODE_JOINT;
  if (!k_txt || !vt_txt || !q_img || !k_img || !vt_img || !o || (joint && !q_txt)) return QI_ERR_NULL;
  if (!al16(k_txt) || !al16(vt_txt) || !al16(q_img) || !al16(k_img) || !al16(vt_img) || !al16(o) ||
      (joint && !al16(q_txt)))
    return QI_ERR_ALIGN;
  return launch_attention(heads, L, N, joint, q_txt, k_txt, vt_txt, q_img, k_img, vt_img, o,
                          (hipStream_t)stream);
}

qi_status qi_linear_bf16(int32_t M, int32_t N, int32_t K, const uint16_t *A, const uint16_t *W,
                         const float *bias, float *C, void *stream) {
  if (M < 1 || N < 128 || N % 128 != 0 || K < 64 || K % 64 != 0 || M > (1 << 20) || N > (1 << 20) ||
      K > (1 << 20))
    return QI_ERR_RANGE;
  if (!A || !W || !C) return QI_ERR_NULL;
  if (!al16(A) || !al16(W) || !al16(C) || (bias && !al16(bias))) return QI_ERR_ALIGN;
  GemmArgs g{};
  g.A = A; g.lda = K; g.W = W; g.ldw = K; g.M = M; g.N = N; g.K = K;
  g.C = C; g.ldc = N; g.bias = bias;
  return launch_gemm<EPI_F32>(g, QI_KERNEL_GEMM_TXT, (hipStream_t)stream);
}

const char *qi_kernel_kind_name(int32_t kind) {
  static const char *names[QI_KERNEL_KINDS] = {"modulation", "txt_norm",   "gemm_txt",  "img_embed",
                                               "norm_mod",   "gemm_qkv",   "attention", "gemm_o",
                                               "gemm_gate_up", "gemm_down", "head",     "euler",
                                               "enc_gemm",   "enc_attention", "enc_misc", "splitk_reduce"};
  return (kind >= 0 && kind < QI_KERNEL_KINDS) ? names[kind] : "?";
}

qi_status qi_timing_begin(int32_t max_launches) {
  if (max_launches < 1 || max_launches > (1 << 20)) return QI_ERR_RANGE;
  std::lock_guard<std::mutex> g(g_timer.mu);
  const size_t need = 2 * (size_t)max_launches;
  while (g_timer.pool.size() < need) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return QI_ERR_HIP;
    g_timer.pool.push_back(e);
  }
  g_timer.kinds.clear();
  g_timer.dropped = 0;
  g_timer.on = true;
  return QI_OK;
}

qi_status qi_timing_end(double *ms_total, int64_t *launches, int64_t *dropped) {
  std::lock_guard<std::mutex> g(g_timer.mu);
  g_timer.on = false;
  if (!ms_total || !launches) return QI_ERR_NULL;
  for (int k = 0; k < QI_KERNEL_KINDS; ++k) {
    ms_total[k] = 0.0;
    launches[k] = 0;
  }
  const size_t n = g_timer.kinds.size();
  if (n && hipEventSynchronize(g_timer.pool[2 * n - 1]) != hipSuccess) return QI_ERR_HIP;
  for (size_t i = 0; i < n; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_timer.pool[2 * i], g_timer.pool[2 * i + 1]) != hipSuccess) return QI_ERR_HIP;
    ms_total[g_timer.kinds[i]] += ms;
    launches[g_timer.kinds[i]] += 1;
  }
  if (dropped) *dropped = (int64_t)g_timer.dropped;
  g_timer.kinds.clear();
  return QI_OK;
}

}  // extern "C"
