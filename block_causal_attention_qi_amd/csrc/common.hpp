// Shared device helpers for the gfx950 (CDNA4) kernels: bf16 packing, MFMA
// operand types and wavefront reductions.  wave64 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define QI_DEV __device__ __forceinline__

QI_DEV float bf16_to_f32(u16 b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
QI_DEV u16 f32_to_bf16(float f) { return __builtin_bit_cast(u16, (__bf16)f); }

// Two fp32 -> one packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32.
QI_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

QI_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D = A(16x32) * B(32x16) + C, bf16 inputs, fp32 accumulate.  Lane l supplies
// A[l%16][8*(l/16) .. +8) and B[8*(l/16) .. +8)[l%16]; D is held as 4 rows
// 4*(l/16) .. +4 of column l%16.
QI_DEV f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// D = A(32x16) * B(16x32) + C, bf16 inputs, fp32 accumulate.  Lane l supplies
// A[l%32][8*(l/32) .. +8) and B[8*(l/32) .. +8)[l%32]; element i of D (16 per
// lane) is row 8*(i/4) + 4*(l/32) + i%4 of column l%32.  On gfx950 the two
// shapes give the same fp32 results bit for bit (measured on MI355X).  In a
// register-only loop this shape reaches about 1.7x the FLOP rate of the
// 16x16x32 one; fed from LDS in the 256 x 256 GEMM tile the 16x16x32 form runs
// faster.
QI_DEV f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// The 4 accumulators 4j .. 4j+3 of a 32x32 MFMA result (rows 8j + 4*(l/32) + 0..3).
QI_DEV f32x4 quad(const f32x16 &a, int j) { return f32x4{a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]}; }

// Exact split of 8 fp32 values into three planes of 8 bf16 (16 bytes each):
// a = a0 + a1 + a2 with a0 = bf16(a), a1 = bf16(a - a0), a2 = a - a0 - a1 (each
// remainder exact in fp32, the last with at most 8 significant bits), so three
// bf16 MFMAs against an exact bf16 operand give the fp32 product sum up to the
// order of the fp32 additions.
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

QI_DEV float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

QI_DEV float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Sum over the whole workgroup (blockDim.x a multiple of 64, <= 1024).
// `red` must hold blockDim.x/64 floats.  Every thread gets the total.
QI_DEV float block_sum(float v, float *red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  __syncthreads();
  return t;
}
