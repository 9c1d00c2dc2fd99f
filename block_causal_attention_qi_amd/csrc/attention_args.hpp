// Arguments and launch shape of the block-causal attention kernel, shared by
// the kernel's translation unit and the host code that launches it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

struct AttnArgs {
  const u16 *q_t, *k_t, *vt_t;  // text segment  (q_t unused when n_txt_qt == 0)
  const u16 *q_i, *k_i, *vt_i;  // image segment
  u16 *o;
  int ldo;                       // heads * 128
  int heads, L, N;
  int ldv_t, ldv_i;              // V^T row strides (>= segment length rounded up to 64)
  int joint;                     // 1: text query tiles too (causal over the text keys)
  int n_img_qt, n_txt_qt;        // query tiles per head (set by launch_block_causal_attn)
  int o_img_row0;                // output row of image query 0 (L in a joint pass, else 0)
  float scale_log2;              // log2(e) / sqrt(128)
  const int *skip;               // first-block cache: when non-NULL and *skip, do nothing
};

namespace attn {
constexpr int BKV = 64;                  // keys per tile
constexpr float RESCALE_SLACK = 8.f;     // log2 units
// A workgroup of WAVES waves takes 32 queries per wave: 8 waves (two per
// SIMD) for the large images, 4 (one per SIMD) when the 8-wave grid would
// leave CUs idle.
template <int WAVES>
struct Shape {
  static constexpr int BQ = WAVES * 32;           // queries per workgroup
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int NLD = BKV * 16 / THREADS;  // 16-byte K (and V^T) chunks per thread per tile
};
}  // namespace attn

// One launch over up to two independent problems of the same shape apart from
// the text segment (true CFG: the positive and the negative prompt's image
// rows, each against its own cached text K/V).  Both must have the same heads,
// N and query-tile counts.
struct AttnBatch {
  AttnArgs br[2];
  int nbranch;  // 1 or 2
};

// Launches the kernel (defined in attention.hip, which is compiled with MFMA
// accumulators in VGPRs) over grid (n_img_qt + n_txt_qt, heads * nbranch),
// choosing the workgroup size and filling in the query-tile counts.  Every
// query's arithmetic is the same in both shapes (one wave walks its 32
// queries over all their keys in one fixed order), so the choice never
// changes a result bit.
void launch_block_causal_attn(const AttnBatch &ab, hipStream_t s);
