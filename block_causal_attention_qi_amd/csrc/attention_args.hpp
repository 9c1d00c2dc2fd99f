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
  int n_img_qt, n_txt_qt;        // query tiles of BQ per head
  int o_img_row0;                // output row of image query 0 (L in a joint pass, else 0)
  float scale_log2;              // log2(e) / sqrt(128)
  const int *skip;               // first-block cache: when non-NULL and *skip, do nothing
};

namespace attn {
constexpr int WAVES = 8;
constexpr int BQ = WAVES * 32;           // queries per workgroup, 32 per wave
constexpr int BKV = 64;
constexpr int THREADS = 64 * WAVES;
constexpr int NLD = BKV * 16 / THREADS;  // 16-byte K (and V^T) chunks per thread per tile
constexpr float RESCALE_SLACK = 8.f;     // log2 units
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
// accumulators in VGPRs) over grid (n_img_qt + n_txt_qt, heads * nbranch).
void launch_block_causal_attn(const AttnBatch &ab, hipStream_t s);
