// Low-rank products of the LoRA branch (lora.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace lsn {

// out(row, j) (+)= scale * sum_k X(row, k) W(k, j) for j < r (r <= 16);
// ext(row, j) = bf16(ext_scale * sum) for j < r and 0 for r <= j < 16.
struct LoraMM {
  const void* X = nullptr;
  int x_f32 = 0;   // X element type: 0 bf16, 1 fp32
  int trans = 0;   // 0: X[row*ldx + k]; 1: X[k*ldx + row]
  int64_t ldx = 0;
  int R = 0, K = 0;
  const float* W = nullptr;  // W(k, j) = W[k*sk + j*sj]
  int64_t sk = 0, sj = 0;
  int r = 0;
  float* out = nullptr;      // out(row, j) at out[row*so_r + j*so_j]; may be null
  int64_t so_r = 0, so_j = 0;
  int accumulate = 0;
  float scale = 1.f;
  uint16_t* ext = nullptr;   // optional bf16 copy
  int64_t ld_ext = 0;
  float ext_scale = 1.f;
  uint32_t xbytes = 0, wbytes = 0;  // set by lora_mm: one block's operand extents
};

// The forward down-projections of all adapted projections of one group,
// which share their input x: t_p = x A_p for p < n, in one launch.
//   x bf16 [R, K] (row stride ldx); AT_p = bf16(A_p)^T [16, K] (rows j >= r
//   zero; lora_at builds it); t_p fp32 [R, r] row-major;
//   ext (may be null) [row, 16 p + j] = bf16(ext_scale t_p(row, j)) for j < r,
//   0 for r <= j < 16.
//   With AF[0] set (n == 1 only), A is read as fp32 [K, r] row-major from
//   AF[0] (rounded to bf16 as it is loaded) and AT is not used.
//   conv (optional): a bf16 row conversion, as lora_ext does, by extra
//   workgroups of the same launch.
struct ExtJob {
  // out[row*ld + c0 + j*oj] = bf16(W[row*srow + j*sj]) for j < r, 0 for
  // r <= j < 16, rows [0, rows); set by the launcher: vec (oj == 1 and every
  // row's 16 outputs are 16-byte aligned) and wbytes (W's extent)
  const float* W = nullptr;
  int64_t srow = 0, sj = 0;
  int rows = 0, r = 0;
  uint16_t* out = nullptr;
  int64_t ld = 0, oj = 1;
  int c0 = 0;
  int vec = 0;
  uint32_t wbytes = 0;
};
// Up to 6 row conversions in one launch (one thread per row).
struct ExtBatch {
  ExtJob job[6];
  int n = 0;
};
hipError_t lora_convert(const ExtBatch& b, hipStream_t s);
// the job of lora_at (AT = bf16(A)^T [16, K] from A fp32 [K, r], rows j >= r
// zero)
ExtJob lora_at_job(const float* A, int K, int r, uint16_t* AT);
struct LoraDown {
  const uint16_t* X = nullptr;
  int64_t ldx = 0;
  int R = 0, K = 0, r = 0, n = 0;
  const uint16_t* AT[3] = {};
  const float* AF[3] = {};
  float* t[3] = {};
  uint16_t* ext = nullptr;
  int64_t ld_ext = 0;
  float ext_scale = 1.f;
  ExtJob conv;
  // optional split-k scratch (lora_down_partial_floats); without it, or too
  // small, one workgroup per 16 rows takes the whole k range
  float* part = nullptr;
  int64_t part_floats = 0;
};
hipError_t lora_down(const LoraDown& a, hipStream_t s);
// floats of split-k scratch lora_down wants for these sizes (0: no split),
// and a bound on it for every R' <= R and every K
int64_t lora_down_partial_floats(int R, int K, int n);
int64_t lora_down_partial_floats_max(int R, int n);

// u_p = dy_p B_p^T for the n adapted projections of one group, in one launch
// (the first step of the branch's backward):
//   dy_p = dy + col0[p] (elements), fp32 or bf16 rows of stride lddy;
//   B_p fp32 [r, N_p];
//   u_p fp32 [R, r] row-major; ext[row, 16 p + j] = bf16(ext_scale u_p(row, j))
//   for j < r and 0 for r <= j < 16.
// Needs N_p % 32 == 0 and 16-byte aligned rows (lora_u_ok).  partial
// (may be null): room for the column-split sums, n * S * R * 16 floats with
// S <= 8 chosen to fit; they are added in a fixed order.
struct LoraU {
  const void* dy = nullptr;
  int dy_f32 = 1;
  int64_t lddy = 0;
  int R = 0, r = 0, n = 0;
  int64_t col0[3] = {};
  int N[3] = {};
  const float* B[3] = {};
  float* u[3] = {};
  uint16_t* ext = nullptr;
  int64_t ld_ext = 0;
  float ext_scale = 1.f;
};
bool lora_u_ok(const LoraU& a);
hipError_t lora_u(const LoraU& a, float* partial, int64_t partial_floats, hipStream_t s);

// Gradients of the adapters as reductions over the tokens m < R:
//   out_z(c, j) (+)= scale * sum_m Y(m, c) Z_z(m, j)     c < C, j < r
// for the nz pairs (Z_z, out_z) of each job, which share the job's Y (fp32 or
// bf16, Y(m, c) = Y[m*ldy + c]).  dA_p += s x^T u_p is one job whose Y is the
// group input x (one pass over x for every adapter of the group); dB_p +=
// s t_p^T dy_p is one job per adapter.  Z_z(m, j) = Z_z[m*ldz + j] (fp32);
// out_z(c, j) at out_z[c*so_c + j*so_j].  No scratch.
struct LoraTGradJob {
  const void* Y = nullptr;
  int C = 0, nz = 0;
  int64_t so_c = 0, so_j = 0;
  const float* Z[3] = {};
  int64_t ldz[3] = {};
  float* out[3] = {};
};
struct LoraTGrad {
  int R = 0, r = 0, y_f32 = 0, njobs = 0;
  int64_t ldy = 0;
  float scale = 1.f;
  int accumulate = 1;
  LoraTGradJob job[3];
  // set by lora_tgrad: tokens per split, splits, partial sums and their
  // offsets per (job, z)
  int tps = 0, nsplit = 1;
  float* part = nullptr;
  int64_t poff[3][3] = {};
};
// part (may be null): scratch for the token-split partial sums; the splits
// (up to 8, about 256 workgroups in all) are limited to what fits, and added
// in split order
hipError_t lora_tgrad(const LoraTGrad& a, float* part, int64_t part_floats, hipStream_t s);

// floats of split-k scratch lora_mm wants for these sizes (0: no split)
int64_t lora_mm_partial_floats(int R, int K);
// partial may be null (then one pass over k)
hipError_t lora_mm(const LoraMM& a, float* partial, int64_t partial_floats, hipStream_t s);

}  // namespace lsn
