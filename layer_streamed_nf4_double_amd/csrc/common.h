// Shared device/host definitions for the gfx950 kernels of liblsn.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LSN_DEV __device__ __forceinline__

LSN_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

LSN_DEV uint16_t f32_to_bf16_bits(float f) {
  bf16 h = (bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, h);
}

LSN_DEV uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (bf16)lo;
  v[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Raw buffer loads: a resource over [base, base + bytes) (base wave-uniform)
// and a per-lane byte offset; offsets at or past the end read 0, so a
// predicated-off element costs no branch (BUF_OOB is past any end).
typedef __amdgpu_buffer_rsrc_t buf_t;
constexpr uint32_t BUF_OOB = 0x80000000u;
LSN_DEV buf_t buf_rsrc(const void* base, uint32_t bytes) {
  // dword 3 = 0x00020000: 32-bit data format (a zero format reads nothing)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
LSN_DEV float buf_f32(buf_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
LSN_DEV uint16_t buf_u16(buf_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
LSN_DEV bf16x8 buf_bf16x8(buf_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// 0 + p[0] + p[stride] + ... + p[(n - 1) stride], added in that order; the
// loads of each group of 8 terms are issued together (n is the same for the
// whole wave, so the tests below are scalar branches, not divergent ones)
LSN_DEV float ordered_sum(const float* __restrict__ p, int64_t stride, int n) {
  float v = 0.f;
  for (int s0 = 0; s0 < n; s0 += 8) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = s0 + e < n ? p[(int64_t)(s0 + e) * stride] : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (s0 + e < n) v += x[e];
  }
  return v;
}

// One row of a bf16 low-rank operand: o[j * oj] = bf16(W[row*srow + j*sj])
// for j < r and 0 for r <= j < 16, W read through the buffer resource w (so
// j >= r reads 0 without a branch).  Threads of consecutive rows read
// consecutive addresses when srow == 1 (a [r, N] matrix turned into [N, 16]
// rows) and write consecutive addresses when oj > 1 (a [K, r] matrix turned
// into [16, K]); vec (oj == 1 only): o is 16-byte aligned (two 16-byte
// stores, else sixteen 2-byte ones).
LSN_DEV void ext_row(buf_t w, int64_t srow, int64_t sj, int64_t row, int r,
                     uint16_t* __restrict__ o, int64_t oj, bool vec) {
  float v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = buf_f32(w, j < r ? (uint32_t)(row * srow + j * sj) * 4 : BUF_OOB);
  uint32_t p[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) p[h] = pack_bf16x2(v[2 * h], v[2 * h + 1]);
  if (vec) {
    reinterpret_cast<u32x4*>(o)[0] = u32x4{p[0], p[1], p[2], p[3]};
    reinterpret_cast<u32x4*>(o)[1] = u32x4{p[4], p[5], p[6], p[7]};
  } else {
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      o[(2 * h) * oj] = (uint16_t)(p[h] & 0xFFFFu);
      o[(2 * h + 1) * oj] = (uint16_t)(p[h] >> 16);
    }
  }
}

// SwiGLU activation silu(g) * u = g * sigmoid(g) * u in fp32.  One definition
// for the stand-alone SwiGLU kernels and the gate|up GEMM epilogue, so both
// give the same bits from the same gate and up values.
LSN_DEV float swiglu_act(float g, float u) { return g * (1.0f / (1.0f + expf(-g))) * u; }

// wave64 reductions in a fixed butterfly order (deterministic)
LSN_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
LSN_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block reduction over up to 1024 threads, fixed order.  `red` must hold
// blockDim.x/64 floats of shared memory.  Result valid in every thread.
LSN_DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}
LSN_DEV float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < nw; ++i) t = fmaxf(t, red[i]);
  return t;
}
