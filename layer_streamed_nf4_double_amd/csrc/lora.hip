// Low-rank (r <= 16) products of the LoRA branch on the matrix cores.
//
//   out(row, j) = scale * sum_k X(row, k) W(k, j)        j < r
//
// X is bf16 or fp32, stored with the reduction contiguous (X[row*ld + k]) or
// transposed (X[k*ld + row]); W(k, j) = W[k*sk + j*sj] is fp32.  This one
// kernel serves the four products of an adapted projection y = xW + s(xA)B:
//   t  = x A            (row = token, k = input feature)
//   u  = dy B^T         (row = token, k = output feature)
//   dA += s x^T u       (row = input feature, k = token; x transposed)
//   dB += s t^T dy      (row = output feature, k = token; dy transposed,
//                        written to dB[j*N + row])
// Operands are rounded to bf16 and multiplied by v_mfma_f32_16x16x32_bf16
// with fp32 accumulation.  One workgroup owns 16 rows; its four waves split
// the k range and are summed in LDS in wave order; with split-k the partial
// sums go to a buffer and a second kernel adds them in split order.  No
// atomics: results are bit-reproducible.
#include "common.h"
#include "lora.h"

namespace lsn {

constexpr int KSTEP = 32;  // k per MFMA

template <bool XF32, bool TRANS>
LSN_DEV float load_x(const void* X, int64_t ldx, int row, int k) {
  const int64_t o = TRANS ? (int64_t)k * ldx + row : (int64_t)row * ldx + k;
  if constexpr (XF32)
    return reinterpret_cast<const float*>(X)[o];
  else
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(X)[o]);
}

LSN_DEV void lora_store(const LoraMM& a, int row, int j, float sum) {
  if (row >= a.R) return;
  if (j < a.r && a.out) {
    float* o = a.out + (int64_t)row * a.so_r + (int64_t)j * a.so_j;
    const float v = a.scale * sum;
    *o = a.accumulate ? *o + v : v;
  }
  if (a.ext) a.ext[(int64_t)row * a.ld_ext + j] = (j < a.r) ? f32_to_bf16_bits(a.ext_scale * sum) : 0;
}

template <bool XF32, bool TRANS>
__global__ __launch_bounds__(256) void lora_mm_k(const LoraMM a, int kchunk, float* partial) {
  __shared__ float red[4][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * 16;
  const int kb = blockIdx.y * kchunk, ke = min(a.K, kb + kchunk);
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int row = row0 + lr;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = kb + wave * KSTEP; k0 < ke; k0 += 4 * KSTEP) {
    bf16x8 af, bw;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + lk + i;
      const bool kin = k < ke;
      af[i] = (bf16)((row < a.R && kin) ? load_x<XF32, TRANS>(a.X, a.ldx, row, k) : 0.f);
      bw[i] = (bf16)((lr < a.r && kin) ? a.W[(int64_t)k * a.sk + (int64_t)lr * a.sj] : 0.f);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bw, acc, 0, 0, 0);
  }
  // lane holds column j = lane % 16, rows (lane / 16) * 4 + i
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][(lane >> 4) * 4 + i][lane & 15] = acc[i];
  __syncthreads();
  const int rr = threadIdx.x >> 4, j = threadIdx.x & 15;
  const float v = ((red[0][rr][j] + red[1][rr][j]) + red[2][rr][j]) + red[3][rr][j];
  if (gridDim.y == 1)
    lora_store(a, row0 + rr, j, v);
  else if (row0 + rr < a.R)
    partial[((int64_t)blockIdx.y * a.R + row0 + rr) * 16 + j] = v;
}

__global__ void lora_reduce_k(const LoraMM a, int nsplit, const float* __restrict__ partial) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.R * 16) return;
  const int row = (int)(i >> 4), j = (int)(i & 15);
  float v = 0.f;
  for (int s = 0; s < nsplit; ++s) v += partial[((int64_t)s * a.R + row) * 16 + j];
  lora_store(a, row, j, v);
}

static void split_of(int R, int K, int* nsplit, int* kchunk) {
  const int rb = (R + 15) / 16;
  int ns = std::max(1, 256 / std::max(rb, 1));
  ns = std::min(ns, std::max(1, (K + 4 * KSTEP - 1) / (4 * KSTEP)));
  ns = std::min(ns, 64);
  int kc = (K + ns - 1) / ns;
  kc = (kc + 4 * KSTEP - 1) / (4 * KSTEP) * (4 * KSTEP);
  *kchunk = std::max(kc, 4 * KSTEP);
  *nsplit = (K + *kchunk - 1) / *kchunk;
}

int64_t lora_mm_partial_floats(int R, int K) {
  int ns, kc;
  split_of(R, K, &ns, &kc);
  return ns > 1 ? (int64_t)ns * R * 16 : 0;
}

// One workgroup of 16 waves owns 16 rows; wave w takes the 32-deep k steps
// w, w + 16, ... for every adapter at once, so each x fragment (one 16-byte
// load where rows are aligned) feeds n MFMAs; the waves' sums are added in
// LDS in wave order.  No split-k: one launch per group.
constexpr int DW = 16;  // waves per workgroup of lora_down_k

template <bool VEC>
__global__ __launch_bounds__(DW * 64) void lora_down_k(const LoraDown a) {
  __shared__ float red[DW][3][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * 16;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int row = row0 + lr;
  const bool rin = row < a.R;
  f32x4 acc[3] = {};
  for (int k0 = wave * KSTEP; k0 < a.K; k0 += DW * KSTEP) {
    bf16x8 xf;
    if (VEC) {
      // K % 8 == 0: a lane's eight columns are all inside the row or all past it
      xf = (rin && k0 + lk < a.K)
               ? *reinterpret_cast<const bf16x8*>(a.X + (int64_t)row * a.ldx + k0 + lk)
               : bf16x8{};
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = k0 + lk + i;
        xf[i] = (bf16)((rin && k < a.K) ? bf16_to_f32(a.X[(int64_t)row * a.ldx + k]) : 0.f);
      }
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      if (q >= a.n) break;
      bf16x8 wf;
      if (VEC) {
        wf = (k0 + lk < a.K) ? *reinterpret_cast<const bf16x8*>(a.AT[q] + (int64_t)lr * a.K + k0 + lk)
                             : bf16x8{};
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = k0 + lk + i;
          wf[i] = (bf16)(k < a.K ? bf16_to_f32(a.AT[q][(int64_t)lr * a.K + k]) : 0.f);
        }
      }
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf, wf, acc[q], 0, 0, 0);
    }
  }
  // lane holds column j = lane % 16, rows (lane / 16) * 4 + i
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][q][(lane >> 4) * 4 + i][lane & 15] = acc[q][i];
  __syncthreads();
  // thread -> (adapter q, row rr, column j)
  const int q = threadIdx.x >> 8, rr = (threadIdx.x >> 4) & 15, j = threadIdx.x & 15;
  const int orow = row0 + rr;
  if (q >= a.n || orow >= a.R) return;
  float v = 0.f;
#pragma unroll
  for (int w = 0; w < DW; ++w) v += red[w][q][rr][j];
  if (j < a.r) a.t[q][(int64_t)orow * a.r + j] = v;
  a.ext[(int64_t)orow * a.ld_ext + 16 * q + j] = (j < a.r) ? f32_to_bf16_bits(a.ext_scale * v) : 0;
}

__global__ void lora_at_k(const float* __restrict__ A, int K, int r, uint16_t* __restrict__ AT) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)16 * K) return;
  const int j = (int)(i / K), k = (int)(i % K);
  AT[i] = j < r ? f32_to_bf16_bits(A[(int64_t)k * r + j]) : 0;
}

void lora_at(const float* A, int K, int r, uint16_t* AT, hipStream_t s) {
  const int64_t n = (int64_t)16 * K;
  hipLaunchKernelGGL(lora_at_k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, A, K, r, AT);
}

hipError_t lora_down(const LoraDown& a, hipStream_t s) {
  if (a.R <= 0 || a.n <= 0) return hipSuccess;
  if (a.n > 3 || a.r > 16) return hipErrorInvalidValue;
  bool vec = a.K % 8 == 0 && a.ldx % 8 == 0 && ((uintptr_t)a.X & 15) == 0;
  for (int q = 0; q < a.n; ++q) vec = vec && ((uintptr_t)a.AT[q] & 15) == 0;
  const dim3 grid((a.R + 15) / 16);
  if (vec) hipLaunchKernelGGL(lora_down_k<true>, grid, dim3(DW * 64), 0, s, a);
  else hipLaunchKernelGGL(lora_down_k<false>, grid, dim3(DW * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t lora_mm(const LoraMM& a, float* partial, int64_t partial_floats, hipStream_t s) {
  if (a.R <= 0) return hipSuccess;
  int ns, kc;
  split_of(a.R, a.K, &ns, &kc);
  if ((int64_t)ns * a.R * 16 > partial_floats || !partial) {  // no room: one pass over k
    ns = 1;
    kc = std::max(a.K, 1);
  }
  const dim3 grid((a.R + 15) / 16, ns);
  if (a.x_f32) {
    if (a.trans)
      hipLaunchKernelGGL((lora_mm_k<true, true>), grid, dim3(256), 0, s, a, kc, partial);
    else
      hipLaunchKernelGGL((lora_mm_k<true, false>), grid, dim3(256), 0, s, a, kc, partial);
  } else {
    if (a.trans)
      hipLaunchKernelGGL((lora_mm_k<false, true>), grid, dim3(256), 0, s, a, kc, partial);
    else
      hipLaunchKernelGGL((lora_mm_k<false, false>), grid, dim3(256), 0, s, a, kc, partial);
  }
  if (ns > 1) {
    const int64_t n = (int64_t)a.R * 16;
    hipLaunchKernelGGL(lora_reduce_k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, ns,
                       partial);
  }
  return hipGetLastError();
}

}  // namespace lsn
