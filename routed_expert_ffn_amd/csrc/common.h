// Device-side helpers shared by the gfx950 kernels of libmoe.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define WAVE 64

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// One OCP e4m3 byte -> fp16 (exact: every finite e4m3 value is an fp16).
__device__ __forceinline__ f16 e4m3_to_f16(uint32_t byte) {
  f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(byte, 1.0f, false);
  return v[0];
}

// Eight e2m1 codes times a power of two: the conversion's scale operand is
// applied through its exponent, which is exact for an MXFP4 block scale
// (the products stay within fp16 for scales within 2^8 .. 2^-23 of 1).
__device__ __forceinline__ f16x8 dequant8_pow2(uint32_t codes, float scale) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 0);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 1);
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 2);
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 3);
  f16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Eight e2m1 codes (one dword, element 0 in the low nibble) times the block
// scale sigma, as eight fp16.  The hardware conversion with a unit scale
// gives the plain e2m1 values; the product e2m1 * e4m3 needs at most six
// significant bits and stays inside fp16's range, so it is exact.
__device__ __forceinline__ f16x8 dequant8(uint32_t codes, f16x2 sigma2) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * sigma2;
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * sigma2;
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * sigma2;
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * sigma2;
  f16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 load_f16x8(const f16* p) { return *reinterpret_cast<const f16x8*>(p); }

// acc += p[s * stride] for s = first .. slabs-1 in ascending order (float4
// partial sums of K slabs), with the loads of eight slabs issued together.
__device__ __forceinline__ void add_slab_partials4(float4& acc, const float* p, long long stride, int first,
                                                   int slabs) {
  for (int s0 = first; s0 < slabs; s0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; u++)
      v[u] = s0 + u < slabs ? *reinterpret_cast<const float4*>(p + (size_t)(s0 + u) * stride)
                            : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int u = 0; u < 8; u++)
      if (s0 + u < slabs) {
        acc.x += v[u].x;
        acc.y += v[u].y;
        acc.z += v[u].z;
        acc.w += v[u].w;
      }
  }
}
