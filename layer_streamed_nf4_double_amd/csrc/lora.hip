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

// ---------------------------------------------------------------------------
// u_p = dy_p B_p^T.  One workgroup of UW waves owns 16 rows of one adapter
// and one of S column ranges; wave w takes the 32-wide column steps w,
// w + UW, ... of its range, each as two 16-byte loads of dy (one for bf16)
// and two of B per lane; the waves' sums are added in LDS in wave order.
// With S > 1 the ranges' sums go to a buffer and lora_u_reduce_k adds them
// in range order.
constexpr int UW = 8;  // waves per workgroup of lora_u_k

struct USplit {
  int S = 1, cols = 0;   // column ranges per adapter and their width (multiple of 32)
  float* part = nullptr;  // [n][S][R][16]
};

template <bool DF32>
__global__ __launch_bounds__(UW * 64) void lora_u_k(const LoraU a, const USplit sp) {
  __shared__ float red[UW][16][17];
  const int q = blockIdx.y, rs = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * 16;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const bool rin = row0 + lr < a.R, jin = lr < a.r;
  const int N = a.N[q];
  const int nb = rs * sp.cols, ne = min(N, nb + sp.cols);
  const int64_t yo = a.col0[q] + (int64_t)(rin ? row0 + lr : 0) * a.lddy + lk;
  const float* B = a.B[q] + (int64_t)(jin ? lr : 0) * N + lk;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int n0 = nb + wave * 32; n0 < ne; n0 += UW * 32) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    bf16x8 af, bw;
    if constexpr (DF32) {
      const float* dy = reinterpret_cast<const float*>(a.dy) + yo + n0;
      const f32x4 x0 = rin ? *reinterpret_cast<const f32x4*>(dy) : zero;
      const f32x4 x1 = rin ? *reinterpret_cast<const f32x4*>(dy + 4) : zero;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = (bf16)x0[i];
        af[i + 4] = (bf16)x1[i];
      }
    } else {
      const uint16_t* dy = reinterpret_cast<const uint16_t*>(a.dy) + yo + n0;
      af = rin ? *reinterpret_cast<const bf16x8*>(dy) : bf16x8{};
    }
    const f32x4 b0 = jin ? *reinterpret_cast<const f32x4*>(B + n0) : zero;
    const f32x4 b1 = jin ? *reinterpret_cast<const f32x4*>(B + n0 + 4) : zero;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bw[i] = (bf16)b0[i];
      bw[i + 4] = (bf16)b1[i];
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bw, acc, 0, 0, 0);
  }
  // lane holds column j = lane % 16, rows (lane / 16) * 4 + i
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][(lane >> 4) * 4 + i][lane & 15] = acc[i];
  __syncthreads();
  if (threadIdx.x >= 256) return;
  const int rr = threadIdx.x >> 4, j = threadIdx.x & 15, row = row0 + rr;
  float v = 0.f;
#pragma unroll
  for (int w = 0; w < UW; ++w) v += red[w][rr][j];
  if (row >= a.R) return;
  if (sp.S > 1) {
    sp.part[(((int64_t)q * sp.S + rs) * a.R + row) * 16 + j] = v;
    return;
  }
  if (j < a.r) a.u[q][(int64_t)row * a.r + j] = v;
  if (a.ext)
    a.ext[(int64_t)row * a.ld_ext + 16 * q + j] = j < a.r ? f32_to_bf16_bits(a.ext_scale * v) : 0;
}

__global__ void lora_u_reduce_k(const LoraU a, const USplit sp) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.n * a.R * 16) return;
  const int q = (int)(i / ((int64_t)a.R * 16));
  const int row = (int)((i >> 4) % a.R), j = (int)(i & 15);
  float v = 0.f;
  for (int s = 0; s < sp.S; ++s) v += sp.part[(((int64_t)q * sp.S + s) * a.R + row) * 16 + j];
  if (j < a.r) a.u[q][(int64_t)row * a.r + j] = v;
  if (a.ext)
    a.ext[(int64_t)row * a.ld_ext + 16 * q + j] = j < a.r ? f32_to_bf16_bits(a.ext_scale * v) : 0;
}

static bool al16(const void* q) { return ((uintptr_t)q & 15) == 0; }

bool lora_u_ok(const LoraU& a) {
  const int v = a.dy_f32 ? 4 : 8;  // elements per 16 bytes
  if (a.n < 1 || a.n > 3 || a.r > 16 || a.lddy % v != 0 || !al16(a.dy)) return false;
  for (int q = 0; q < a.n; ++q)
    if (a.N[q] % 32 != 0 || a.col0[q] % v != 0 || !al16(a.B[q])) return false;
  return true;
}

hipError_t lora_u(const LoraU& a, float* partial, int64_t partial_floats, hipStream_t s) {
  if (a.R <= 0 || a.n <= 0) return hipSuccess;
  if (!lora_u_ok(a)) return hipErrorInvalidValue;
  // column ranges of >= 512 so that ~256 workgroups stream dy (one range
  // when the buffer is missing or too small)
  int nmax = 0;
  for (int q = 0; q < a.n; ++q) nmax = std::max(nmax, a.N[q]);
  const int rb = (a.R + 15) / 16;
  USplit sp;
  sp.S = std::max(1, std::min({8, nmax / 512, 256 / std::max(1, rb * a.n)}));
  while (sp.S > 1 && (!partial || (int64_t)a.n * sp.S * a.R * 16 > partial_floats)) --sp.S;
  sp.cols = ((nmax + sp.S - 1) / sp.S + 31) / 32 * 32;
  sp.part = partial;
  const dim3 grid(rb, a.n, sp.S);
  if (a.dy_f32) hipLaunchKernelGGL(lora_u_k<true>, grid, dim3(UW * 64), 0, s, a, sp);
  else hipLaunchKernelGGL(lora_u_k<false>, grid, dim3(UW * 64), 0, s, a, sp);
  if (sp.S > 1) {
    const int64_t n = (int64_t)a.n * a.R * 16;
    hipLaunchKernelGGL(lora_u_reduce_k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, sp);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Adapter gradients.  A workgroup of 4 waves owns 64 columns c of one job.
// Per block of TB tokens it loads Y [TB x 64] and every Z_z [TB x 16] in one
// burst (16-byte loads where the row allows), rounds them to bf16 and stores
// them transposed in LDS (column-major in m), so that each MFMA fragment --
// 8 consecutive tokens of one column -- is one 16-byte LDS read; wave w then
// runs the block's MFMAs for its 16 columns.  With few column blocks the
// tokens are split over blockIdx.z (up to 8 ranges); each range's sum is one
// lane's in token order and lora_tgrad_reduce_k adds the ranges in order:
// deterministic.
constexpr int TB = 256;      // tokens per LDS block
constexpr int TBP = TB + 8;  // padded row (bf16) of the transposed tiles

template <bool YF32>
__global__ __launch_bounds__(256) void lora_tgrad_k(const LoraTGrad a) {
  __shared__ __attribute__((aligned(16))) uint16_t sY[64][TBP];
  __shared__ __attribute__((aligned(16))) uint16_t sZ[3][16][TBP];
  const LoraTGradJob& jb = a.job[blockIdx.y];
  const int c0 = blockIdx.x * 64;
  if (c0 >= jb.C) return;  // uniform over the workgroup
  // token range of this split (blockIdx.z)
  const int mlo = blockIdx.z * a.tps, mhi = min(a.R, mlo + a.tps);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nz = jb.nz;
  f32x4 acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // staging map: thread t takes 8 consecutive columns cc of token rows
  // t / 8 + 32 i of the block; Z entries: token t / 8 + 32 i, j pair 2 (t % 8)
  const int cc = (t & 7) * 8, mr = t >> 3;
  const bool cfull = c0 + cc + 8 <= jb.C;
  const bool yvec = cfull && (a.ldy % (YF32 ? 4 : 8)) == 0 &&
                    ((uintptr_t)jb.Y & 15) == 0 && ((c0 + cc) % (YF32 ? 4 : 8)) == 0;
  for (int mb = mlo; mb < mhi; mb += TB) {
    // every load of the block first (one round trip), then bf16 + LDS
    constexpr int NI = TB / 32;
    float v[NI][8];
    float zv[3][NI][2];
    if (yvec) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int m = mb + mr + 32 * i;
        const bool in = m < mhi;
        if constexpr (YF32) {
          const float* y = reinterpret_cast<const float*>(jb.Y) + (int64_t)(in ? m : 0) * a.ldy + c0 + cc;
          const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
          const f32x4 y0 = in ? *reinterpret_cast<const f32x4*>(y) : zero;
          const f32x4 y1 = in ? *reinterpret_cast<const f32x4*>(y + 4) : zero;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[i][e] = y0[e];
            v[i][e + 4] = y1[e];
          }
        } else {
          const uint16_t* y =
              reinterpret_cast<const uint16_t*>(jb.Y) + (int64_t)(in ? m : 0) * a.ldy + c0 + cc;
          const u32x4 zero = {0u, 0u, 0u, 0u};
          const u32x4 w4 = in ? *reinterpret_cast<const u32x4*>(y) : zero;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[i][2 * e] = bf16_to_f32((uint16_t)(w4[e] & 0xffff));
            v[i][2 * e + 1] = bf16_to_f32((uint16_t)(w4[e] >> 16));
          }
        }
      }
    } else {  // ragged column block or unaligned rows
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int m = mb + mr + 32 * i;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = c0 + cc + e;
          float y = 0.f;
          if (m < mhi && c < jb.C) {
            const int64_t o = (int64_t)m * a.ldy + c;
            if constexpr (YF32) y = reinterpret_cast<const float*>(jb.Y)[o];
            else y = bf16_to_f32(reinterpret_cast<const uint16_t*>(jb.Y)[o]);
          }
          v[i][e] = y;
        }
      }
    }
    const int jz = 2 * (t & 7);
#pragma unroll
    for (int z = 0; z < 3; ++z) {
      if (z >= nz) break;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int m = mb + mr + 32 * i;
        const float* zr = jb.Z[z] + (int64_t)(m < mhi ? m : 0) * jb.ldz[z];
        zv[z][i][0] = (m < mhi && jz < a.r) ? zr[jz] : 0.f;
        zv[z][i][1] = (m < mhi && jz + 1 < a.r) ? zr[jz + 1] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int ml = mr + 32 * i;
#pragma unroll
      for (int e = 0; e < 8; ++e) sY[cc + e][ml] = f32_to_bf16_bits(v[i][e]);
#pragma unroll
      for (int z = 0; z < 3; ++z) {
        if (z >= nz) break;
        sZ[z][jz][ml] = f32_to_bf16_bits(zv[z][i][0]);
        sZ[z][jz + 1][ml] = f32_to_bf16_bits(zv[z][i][1]);
      }
    }
    __syncthreads();
    const int nk = min(TB, mhi - mb);
    for (int k0 = 0; k0 < nk; k0 += 32) {
      const int kk = k0 + (lane >> 4) * 8;
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(&sY[16 * wave + (lane & 15)][kk]);
#pragma unroll
      for (int z = 0; z < 3; ++z) {
        if (z >= nz) break;
        const bf16x8 bz = *reinterpret_cast<const bf16x8*>(&sZ[z][lane & 15][kk]);
        acc[z] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bz, acc[z], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // lane holds C[c = 16 wave + 4 (lane / 16) + i][j = lane % 16]
  const int j = lane & 15;
  if (j >= a.r) return;
#pragma unroll
  for (int z = 0; z < 3; ++z) {
    if (z >= nz) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + 16 * wave + 4 * (lane >> 4) + i;
      if (c >= jb.C) continue;
      if (a.nsplit > 1) {  // raw sum of this token range, added by lora_tgrad_reduce_k
        a.part[a.poff[blockIdx.y][z] + ((int64_t)blockIdx.z * jb.C + c) * 16 + j] = acc[z][i];
        continue;
      }
      float* o = jb.out[z] + (int64_t)c * jb.so_c + (int64_t)j * jb.so_j;
      const float v = a.scale * acc[z][i];
      *o = a.accumulate ? *o + v : v;
    }
  }
}

// out(c, j) (+)= scale * (sum over the token splits, in split order, of the
// partial sums); blockIdx.y = job * 3 + z
__global__ __launch_bounds__(256) void lora_tgrad_reduce_k(const LoraTGrad a) {
  const int q = blockIdx.y / 3, z = blockIdx.y % 3;
  const LoraTGradJob& jb = a.job[q];
  if (z >= jb.nz) return;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // c * 16 + j
  if (e >= (int64_t)jb.C * 16) return;
  const int c = (int)(e >> 4), j = (int)(e & 15);
  if (j >= a.r) return;
  const float* pp = a.part + a.poff[q][z] + e;
  float sum = 0.f;
  for (int sp = 0; sp < a.nsplit; ++sp) sum += pp[(int64_t)sp * jb.C * 16];
  float* o = jb.out[z] + (int64_t)c * jb.so_c + (int64_t)j * jb.so_j;
  const float v = a.scale * sum;
  *o = a.accumulate ? *o + v : v;
}

hipError_t lora_tgrad(const LoraTGrad& a0, float* part, int64_t part_floats, hipStream_t s) {
  LoraTGrad a = a0;
  if (a.R <= 0 || a.njobs <= 0) return hipSuccess;
  if (a.njobs > 3 || a.r > 16) return hipErrorInvalidValue;
  int cmax = 0;
  int64_t per_split = 0;  // partial-sum floats of one token split
  for (int q = 0; q < a.njobs; ++q) {
    if (a.job[q].nz < 1 || a.job[q].nz > 3) return hipErrorInvalidValue;
    cmax = std::max(cmax, a.job[q].C);
    per_split += (int64_t)a.job[q].nz * a.job[q].C * 16;
  }
  // token splits: about 256 workgroups, at least 64 tokens per split, and
  // the partial sums within the scratch (else one pass over the tokens)
  const int wgs = ((cmax + 63) / 64) * a.njobs;
  int ns = std::max(1, std::min({8, 256 / std::max(wgs, 1), a.R / 64}));
  if (!part) ns = 1;
  while (ns > 1 && per_split * ns > part_floats) --ns;
  a.tps = ((a.R + ns - 1) / ns + 31) / 32 * 32;
  a.nsplit = (a.R + a.tps - 1) / a.tps;
  a.part = part;
  if (a.nsplit > 1) {
    int64_t off = 0;
    for (int q = 0; q < a.njobs; ++q)
      for (int z = 0; z < a.job[q].nz; ++z) {
        a.poff[q][z] = off;
        off += (int64_t)a.nsplit * a.job[q].C * 16;
      }
  }
  const dim3 grid((cmax + 63) / 64, a.njobs, a.nsplit);
  if (a.y_f32) hipLaunchKernelGGL(lora_tgrad_k<true>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(lora_tgrad_k<false>, grid, dim3(256), 0, s, a);
  if (a.nsplit > 1)
    hipLaunchKernelGGL(lora_tgrad_reduce_k, dim3((cmax * 16 + 255) / 256, a.njobs * 3), dim3(256), 0,
                       s, a);
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
