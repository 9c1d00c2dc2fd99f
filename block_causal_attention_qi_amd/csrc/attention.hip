// Translation unit of the attention kernel.  It is compiled with
// -amdgpu-mfma-vgpr-form: with two waves per SIMD and 256 registers each, the
// score and output accumulators must share the VGPR file with the softmax
// state; in the default (AGPR) form the compiler spills.
#include "attention.hpp"

// 8-wave workgroups when they give every CU one, else 4-wave ones: a wave's
// walk over its keys sets the launch time, and one wave per SIMD walks
// faster than two sharing it (384^2: 37.6 -> 28.8 us; at 1024^2 the 4-wave
// grid is 32% slower, so it is kept for small grids only).
template <int WAVES>
void launch_shape(AttnBatch ab, hipStream_t s) {
  constexpr int BQ = attn::Shape<WAVES>::BQ;
  for (int b = 0; b < ab.nbranch; ++b) {
    AttnArgs &a = ab.br[b];
    a.n_img_qt = (a.N + BQ - 1) / BQ;
    a.n_txt_qt = a.joint ? (a.L + BQ - 1) / BQ : 0;
  }
  const AttnArgs &a = ab.br[0];
  hipLaunchKernelGGL(block_causal_attn_kernel<WAVES>, dim3(a.n_img_qt + a.n_txt_qt, a.heads * ab.nbranch),
                     dim3(attn::Shape<WAVES>::THREADS), 0, s, ab);
}

void launch_block_causal_attn(const AttnBatch &ab, hipStream_t s) {
  const AttnArgs &a = ab.br[0];
  constexpr int BQ8 = attn::Shape<8>::BQ;
  const int wgs8 = ((a.N + BQ8 - 1) / BQ8 + (a.joint ? (a.L + BQ8 - 1) / BQ8 : 0)) * a.heads * ab.nbranch;
  if (wgs8 >= 256)
    launch_shape<8>(ab, s);
  else
    launch_shape<4>(ab, s);
}
