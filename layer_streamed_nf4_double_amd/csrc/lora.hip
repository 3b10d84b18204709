// Low-rank (r <= 16) products of the LoRA branch y = xW + s(xA)B on the
// matrix cores:
//   t  = x A            lora_down_k (every adapter of a projection group)
//   u  = dy B^T         lora_u_k
//   dA += s x^T u,  dB += s t^T dy    lora_tgrad_k
// and lora_mm_k, the general product
//   out(row, j) = scale * sum_k X(row, k) W(k, j)        j < r
// with X bf16 or fp32, stored with the reduction contiguous (X[row*ld + k])
// or transposed (X[k*ld + row]) and W(k, j) = W[k*sk + j*sj] fp32, for the
// operands the others do not take (rows not 16-byte aligned);
// lora_convert_k writes the bf16 adapter copies the GEMMs read as extra
// k-columns.  Operands are rounded to bf16 and multiplied by
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  The sums of waves, and
// of the k splits of a split launch, are added in fixed orders; no atomics:
// results are bit-reproducible.
//
// These launches have few workgroups each, so they are bound by load
// latency: operands are read through raw buffer loads (an element outside
// its operand reads 0, without a branch) and a wave issues several k steps'
// loads before their MFMAs.
#include "common.h"
#include "lora.h"

namespace lsn {

constexpr int KSTEP = 32;  // k per MFMA

LSN_DEV void lora_store(const LoraMM& a, int row, int j, float sum) {
  if (row >= a.R) return;
  if (j < a.r && a.out) {
    float* o = a.out + (int64_t)row * a.so_r + (int64_t)j * a.so_j;
    const float v = a.scale * sum;
    *o = a.accumulate ? *o + v : v;
  }
  if (a.ext) a.ext[(int64_t)row * a.ld_ext + j] = (j < a.r) ? f32_to_bf16_bits(a.ext_scale * sum) : 0;
}

// lora_mm_k: one workgroup owns 16 rows; its four waves take the 32-deep k
// steps w, w + 4, ... of the block's k range and are summed in LDS in wave
// order; with a split launch the partial sums go to a buffer and
// lora_reduce_k adds them in split order.
template <bool XF32, bool TRANS>
__global__ __launch_bounds__(256) void lora_mm_k(const LoraMM a, int kchunk, float* partial) {
  __shared__ float red[4][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * 16;
  const int kb = blockIdx.y * kchunk, ke = min(a.K, kb + kchunk);
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const bool rin = row0 + lr < a.R, jin = lr < a.r;
  // buffer loads over this block's part of X and W (an element outside the
  // rows, the k range or the r columns reads 0, with no branch); the loads
  // of NB k steps are issued before their MFMAs, which run in k order
  constexpr int ES = XF32 ? 4 : 2;
  const char* xb = reinterpret_cast<const char*>(a.X) +
                   (TRANS ? (int64_t)kb * a.ldx + row0 : (int64_t)row0 * a.ldx + kb) * ES;
  const buf_t xr = buf_rsrc(xb, a.xbytes);
  const buf_t wr = buf_rsrc(a.W + (int64_t)kb * a.sk, a.wbytes);
  constexpr int NB = 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int kq = kb + wave * KSTEP; kq < ke; kq += NB * 4 * KSTEP) {
    float xv[NB][8], wv[NB][8];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = kq + u * 4 * KSTEP + lk + i;
        const int64_t kl = k - kb;
        const uint32_t xo = rin && k < ke
                                ? (uint32_t)((TRANS ? kl * a.ldx + lr : (int64_t)lr * a.ldx + kl) * ES)
                                : BUF_OOB;
        xv[u][i] = XF32 ? buf_f32(xr, xo) : bf16_to_f32(buf_u16(xr, xo));
        wv[u][i] = buf_f32(wr, jin && k < ke ? (uint32_t)((kl * a.sk + (int64_t)lr * a.sj) * 4)
                                             : BUF_OOB);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (kq + u * 4 * KSTEP >= ke) break;  // the same for the whole wave
      bf16x8 af, bw;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        af[i] = (bf16)xv[u][i];
        bw[i] = (bf16)wv[u][i];
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bw, acc, 0, 0, 0);
    }
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
  const float v = ordered_sum(partial + (int64_t)row * 16 + j, (int64_t)a.R * 16, nsplit);
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
// LDS in wave order.  No split-k: one launch per group.  The launch has few
// workgroups, so it is bound by load latency, not bandwidth: a wave issues
// the loads of DB k steps (2 where it loads element by element) before their
// MFMAs, which still run in k order.  Workgroups past the row blocks do the
// launch's row conversion (ExtJob), one row per thread.
constexpr int DW = 16;  // waves per workgroup of lora_down_k
constexpr int DB = 4;   // k steps per batch of loads

LSN_DEV void conv_row(const ExtJob& c, int64_t row) {
  if (row < c.rows)
    ext_row(buf_rsrc(c.W, c.wbytes), c.srow, c.sj, row, c.r, c.out + row * c.ld + c.c0, c.oj,
            c.vec);
}

// blockIdx.y: the k range [y kchunk, (y + 1) kchunk) of a split launch, whose
// sums go to part (lora_down_reduce_k adds them in split order)
template <bool VEC, bool AF32>
__global__ __launch_bounds__(DW * 64) void lora_down_k(const LoraDown a, int nrb, int kchunk,
                                                       float* __restrict__ part) {
  __shared__ float red[DW][3][16][17];
  if ((int)blockIdx.x >= nrb) {
    conv_row(a.conv, (int64_t)(blockIdx.x - nrb) * (DW * 64) + threadIdx.x);
    return;
  }
  const int kbeg = blockIdx.y * kchunk, kend = min(a.K, kbeg + kchunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * 16;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const bool jin = lr < a.r;
  constexpr int NQ = AF32 ? 1 : 3;   // adapters (fp32 A: one)
  constexpr int NB = VEC ? DB : 2;  // element-wise loads: fewer in flight
  // Buffer loads: an element outside its operand reads 0 with no branch (a
  // load under a divergent branch is waited for before the branch joins,
  // which would serialize the batch).  X's resource covers this block's rows,
  // so lanes past the last row read past its end.
  const int nrow = min(16, a.R - row0);
  const buf_t xr = buf_rsrc(a.X + (int64_t)row0 * a.ldx, (uint32_t)(nrow * a.ldx * 2));
  const uint32_t xo = (uint32_t)(lr * a.ldx) * 2;
  buf_t wr[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    wr[q] = AF32 ? buf_rsrc(a.AF[q], (uint32_t)(a.K * a.r) * 4)
                 : buf_rsrc(q < a.n ? a.AT[q] : a.AT[0], (uint32_t)(16 * a.K) * 2);
  f32x4 acc[3] = {};
  for (int kb = kbeg + wave * KSTEP; kb < kend; kb += NB * DW * KSTEP) {
    // all loads of the batch first (raw values), then the conversions and
    // MFMAs: the scheduling barrier keeps the compiler from interleaving
    // them, which would wait for each k step's loads in turn
    bf16x8 xf[NB], wf[NB][3];
    float af[NB][8];                   // fp32 A
    uint16_t xs[NB][8], ws[NB][3][8];  // element-wise loads
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int k0 = kb + u * DW * KSTEP;
      // VEC: K and the k ranges are multiples of 8, so a lane's eight
      // columns are all inside the range or all past it
      const bool kin8 = k0 + lk < kend;
      if (VEC) {
        xf[u] = buf_bf16x8(xr, kin8 ? xo + (uint32_t)(k0 + lk) * 2 : BUF_OOB);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = k0 + lk + i;
          xs[u][i] = buf_u16(xr, k < kend ? xo + (uint32_t)k * 2 : BUF_OOB);
        }
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (!AF32 && q >= a.n) break;  // fp32 A: n == 1
        if (AF32) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int k = k0 + lk + i;
            af[u][i] = buf_f32(wr[q], jin && k < kend ? (uint32_t)(k * a.r + lr) * 4 : BUF_OOB);
          }
        } else if (VEC) {
          wf[u][q] = buf_bf16x8(wr[q], kin8 ? (uint32_t)(lr * a.K + k0 + lk) * 2 : BUF_OOB);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int k = k0 + lk + i;
            ws[u][q][i] = buf_u16(wr[q], k < kend ? (uint32_t)(lr * a.K + k) * 2 : BUF_OOB);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (!VEC) xf[u][i] = __builtin_bit_cast(bf16, xs[u][i]);
        if (AF32) wf[u][0][i] = (bf16)af[u][i];
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (!AF32 && q >= a.n) break;
        if (!AF32 && !VEC)
#pragma unroll
          for (int i = 0; i < 8; ++i) wf[u][q][i] = __builtin_bit_cast(bf16, ws[u][q][i]);
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[u], wf[u][q], acc[q], 0, 0, 0);
      }
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
  if (gridDim.y > 1) {
    part[(((int64_t)blockIdx.y * a.n + q) * a.R + orow) * 16 + j] = v;
    return;
  }
  if (j < a.r) a.t[q][(int64_t)orow * a.r + j] = v;
  if (a.ext)
    a.ext[(int64_t)orow * a.ld_ext + 16 * q + j] = (j < a.r) ? f32_to_bf16_bits(a.ext_scale * v) : 0;
}

// the launcher's fields of a conversion job; false if W's extent does not
// fit the 32-bit offsets of the buffer loads
static bool prep_job(ExtJob& c) {
  c.vec = c.oj == 1 && c.ld % 8 == 0 && c.c0 % 8 == 0 && ((uintptr_t)c.out & 15) == 0;
  const int64_t ext =
      c.rows > 0 && c.r > 0 ? ((int64_t)(c.rows - 1) * c.srow + (int64_t)(c.r - 1) * c.sj + 1) * 4 : 0;
  if (ext >= BUF_OOB) return false;
  c.wbytes = (uint32_t)ext;
  return true;
}

__global__ __launch_bounds__(256) void lora_convert_k(const ExtBatch b) {
  const ExtJob& c = b.job[blockIdx.y];
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row < c.rows)
    ext_row(buf_rsrc(c.W, c.wbytes), c.srow, c.sj, row, c.r, c.out + row * c.ld + c.c0, c.oj,
            c.vec);
}

hipError_t lora_convert(const ExtBatch& b0, hipStream_t s) {
  if (b0.n < 0 || b0.n > 6) return hipErrorInvalidValue;
  ExtBatch b = b0;
  int rmax = 0;
  for (int i = 0; i < b.n; ++i) {
    if (b.job[i].r < 0 || b.job[i].r > 16 || !prep_job(b.job[i])) return hipErrorInvalidValue;
    rmax = std::max(rmax, b.job[i].rows);
  }
  if (b.n == 0 || rmax <= 0) return hipSuccess;
  hipLaunchKernelGGL(lora_convert_k, dim3((unsigned)((rmax + 255) / 256), b.n), dim3(256), 0, s, b);
  return hipGetLastError();
}

ExtJob lora_at_job(const float* A, int K, int r, uint16_t* AT) {
  // row k of the job is column k of AT: AT[j*K + k] = bf16(A[k*r + j])
  return ExtJob{A, r, 1, K, r, AT, 1, K, 0, 0};
}

// the split sums of a split lora_down_k, added in split order; workgroups
// past nred do the launch's row conversion
__global__ __launch_bounds__(256) void lora_down_reduce_k(const LoraDown a, int ns, int nred,
                                                          const float* __restrict__ part) {
  if ((int)blockIdx.x >= nred) {
    conv_row(a.conv, (int64_t)(blockIdx.x - nred) * 256 + threadIdx.x);
    return;
  }
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (q, row, j)
  if (i >= (int64_t)a.n * a.R * 16) return;
  const int q = (int)(i / ((int64_t)a.R * 16)), j = (int)(i & 15);
  const int64_t row = (i >> 4) % a.R;
  const float v = ordered_sum(part + i, (int64_t)a.n * a.R * 16, ns);
  if (j < a.r) a.t[q][row * a.r + j] = v;
  if (a.ext) a.ext[row * a.ld_ext + 16 * q + j] = (j < a.r) ? f32_to_bf16_bits(a.ext_scale * v) : 0;
}

// k split of lora_down: about 256 workgroups, at least DW k steps per split
static void down_split(int R, int K, int* ns, int* kchunk) {
  const int nrb = (R + 15) / 16;
  int s = std::max(1, std::min({8, 256 / std::max(nrb, 1), (K + DW * KSTEP - 1) / (DW * KSTEP)}));
  int kc = (K + s - 1) / s;
  kc = (kc + DW * KSTEP - 1) / (DW * KSTEP) * (DW * KSTEP);
  *kchunk = kc;
  *ns = (K + kc - 1) / kc;
}

int64_t lora_down_partial_floats(int R, int K, int n) {
  int ns, kc;
  down_split(R, K, &ns, &kc);
  return ns > 1 ? (int64_t)ns * n * R * 16 : 0;
}

int64_t lora_down_partial_floats_max(int R, int n) { return (int64_t)8 * n * R * 16; }

hipError_t lora_down(const LoraDown& a, hipStream_t s) {
  if (a.n < 0 || a.n > 3 || a.r > 16 || (a.n > 0 && a.R > 0 && a.r <= 0)) return hipErrorInvalidValue;
  const bool af32 = a.n > 0 && a.AF[0] != nullptr;
  if (af32 && a.n != 1) return hipErrorInvalidValue;
  // byte offsets of the buffer loads are 32-bit
  if ((int64_t)16 * a.ldx * 2 >= BUF_OOB || (int64_t)16 * a.K * 4 >= BUF_OOB)
    return hipErrorInvalidValue;
  bool vec = a.K % 8 == 0 && a.ldx % 8 == 0 && ((uintptr_t)a.X & 15) == 0;
  for (int q = 0; q < a.n; ++q)
    vec = vec && (af32 ? a.AF[q] != nullptr : ((uintptr_t)a.AT[q] & 15) == 0);
  const int nrb = a.n > 0 && a.R > 0 ? (a.R + 15) / 16 : 0;
  const int ncb = a.conv.rows > 0 ? (a.conv.rows + DW * 64 - 1) / (DW * 64) : 0;
  if (nrb + ncb == 0) return hipSuccess;
  LoraDown b = a;
  if (b.conv.r < 0 || b.conv.r > 16 || !prep_job(b.conv)) return hipErrorInvalidValue;
  int ns = 1, kc = std::max(a.K, 1);
  if (nrb > 0 && a.part) {
    down_split(a.R, a.K, &ns, &kc);
    if ((int64_t)ns * a.n * a.R * 16 > a.part_floats) ns = 1, kc = std::max(a.K, 1);
  }
  // unsplit: the row conversion rides on this launch; split: on the reduction's
  const dim3 grid(ns > 1 ? nrb : nrb + ncb, ns), blk(DW * 64);
  if (af32) {
    if (vec) hipLaunchKernelGGL((lora_down_k<true, true>), grid, blk, 0, s, b, nrb, kc, a.part);
    else hipLaunchKernelGGL((lora_down_k<false, true>), grid, blk, 0, s, b, nrb, kc, a.part);
  } else {
    if (vec) hipLaunchKernelGGL((lora_down_k<true, false>), grid, blk, 0, s, b, nrb, kc, a.part);
    else hipLaunchKernelGGL((lora_down_k<false, false>), grid, blk, 0, s, b, nrb, kc, a.part);
  }
  if (ns > 1) {
    const int nred = (int)(((int64_t)a.n * a.R * 16 + 255) / 256);
    const int ncr = a.conv.rows > 0 ? (a.conv.rows + 255) / 256 : 0;
    hipLaunchKernelGGL(lora_down_reduce_k, dim3(nred + ncr), dim3(256), 0, s, b, ns, nred,
                       (const float*)a.part);
  }
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
  const bool jin = lr < a.r;
  const int N = a.N[q];
  const int nb = rs * sp.cols, ne = min(N, nb + sp.cols);
  // buffer loads (an element outside reads 0, no branch): dy over this
  // block's rows from column col0, B over its r rows; the loads of UB
  // column steps are issued before their MFMAs, which run in column order
  constexpr int ES = DF32 ? 4 : 2;  // bytes per dy element
  const int nrow = min(16, a.R - row0);
  const buf_t yr = buf_rsrc(reinterpret_cast<const char*>(a.dy) +
                                (a.col0[q] + (int64_t)row0 * a.lddy) * ES,
                            (uint32_t)(nrow * a.lddy * ES));
  const buf_t br = buf_rsrc(a.B[q], (uint32_t)(a.r * N) * 4);
  const uint32_t yo = (uint32_t)(lr * a.lddy + lk) * ES;
  const uint32_t bo = jin ? (uint32_t)(lr * N + lk) * 4 : BUF_OOB;
  constexpr int UB = 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int nb0 = nb + wave * 32; nb0 < ne; nb0 += UB * UW * 32) {
    // N and the ranges are multiples of 32: a step is all inside or all past
    f32x4 x[UB][2], b[UB][2];
    bf16x8 xb[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int n0 = nb0 + u * UW * 32;
      const bool in = n0 < ne;
      if constexpr (DF32) {
        x[u][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                yr, (int)(in ? yo + n0 * ES : BUF_OOB), 0, 0));
        x[u][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                yr, (int)(in ? yo + (n0 + 4) * ES : BUF_OOB), 0, 0));
      } else {
        xb[u] = buf_bf16x8(yr, in ? yo + n0 * ES : BUF_OOB);
      }
      const uint32_t o = in && jin ? bo + n0 * 4 : BUF_OOB;
      b[u][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(br, (int)o, 0, 0));
      b[u][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              br, (int)(o == BUF_OOB ? o : o + 16), 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if (nb0 + u * UW * 32 >= ne) break;
      bf16x8 af, bw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (DF32) {
          af[i] = (bf16)x[u][0][i];
          af[i + 4] = (bf16)x[u][1][i];
        }
        bw[i] = (bf16)b[u][0][i];
        bw[i + 4] = (bf16)b[u][1][i];
      }
      if constexpr (!DF32) af = xb[u];
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bw, acc, 0, 0, 0);
    }
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
  const float v = ordered_sum(sp.part + ((int64_t)q * sp.S * a.R + row) * 16 + j,
                              (int64_t)a.R * 16, sp.S);
  if (j < a.r) a.u[q][(int64_t)row * a.r + j] = v;
  if (a.ext)
    a.ext[(int64_t)row * a.ld_ext + 16 * q + j] = j < a.r ? f32_to_bf16_bits(a.ext_scale * v) : 0;
}

static bool al16(const void* q) { return ((uintptr_t)q & 15) == 0; }

bool lora_u_ok(const LoraU& a) {
  const int v = a.dy_f32 ? 4 : 8;  // elements per 16 bytes
  if (a.n < 1 || a.n > 3 || a.r > 16 || a.lddy % v != 0 || !al16(a.dy)) return false;
  // 32-bit byte offsets of the buffer loads
  if ((int64_t)16 * a.lddy * 4 >= BUF_OOB) return false;
  for (int q = 0; q < a.n; ++q)
    if (a.N[q] % 32 != 0 || a.col0[q] % v != 0 || !al16(a.B[q]) ||
        (int64_t)16 * a.N[q] * 4 >= BUF_OOB)
      return false;
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
  constexpr int ES = YF32 ? 4 : 2;  // bytes per Y element
  const int jz = 2 * (t & 7);
  for (int mb = mlo; mb < mhi; mb += TB) {
    // every load of the block first (one round trip), then bf16 + LDS.
    // Buffer loads over the block's token rows: an element past the last
    // row or column, or a Z column j >= r, reads 0 with no branch
    constexpr int NI = TB / 32;
    const int nm = min(TB, mhi - mb);
    const buf_t yr = buf_rsrc(reinterpret_cast<const char*>(jb.Y) + (int64_t)mb * a.ldy * ES,
                              (uint32_t)((int64_t)nm * a.ldy * ES));
    float v[NI][8];
    float zv[3][NI][2];
    if (yvec) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int ml = mr + 32 * i;
        const uint32_t o = (uint32_t)((int64_t)ml * a.ldy + c0 + cc) * ES;
        if constexpr (YF32) {
          const f32x4 y0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(yr, (int)o, 0, 0));
          const f32x4 y1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(yr, (int)(o + 16), 0, 0));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[i][e] = y0[e];
            v[i][e + 4] = y1[e];
          }
        } else {
          const u32x4 w4 = __builtin_amdgcn_raw_buffer_load_b128(yr, (int)o, 0, 0);
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
        const int ml = mr + 32 * i;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = c0 + cc + e;
          const uint32_t o = c < jb.C ? (uint32_t)((int64_t)ml * a.ldy + c) * ES : BUF_OOB;
          if constexpr (YF32) v[i][e] = buf_f32(yr, o);
          else v[i][e] = bf16_to_f32(buf_u16(yr, o));
        }
      }
    }
#pragma unroll
    for (int z = 0; z < 3; ++z) {
      if (z >= nz) break;
      const buf_t zr = buf_rsrc(jb.Z[z] + (int64_t)mb * jb.ldz[z], (uint32_t)(nm * jb.ldz[z]) * 4);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const uint32_t o = (uint32_t)((mr + 32 * i) * jb.ldz[z] + jz) * 4;
        zv[z][i][0] = buf_f32(zr, jz < a.r ? o : BUF_OOB);
        zv[z][i][1] = buf_f32(zr, jz + 1 < a.r ? o + 4 : BUF_OOB);
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
  const float sum = ordered_sum(pp, (int64_t)jb.C * 16, a.nsplit);
  float* o = jb.out[z] + (int64_t)c * jb.so_c + (int64_t)j * jb.so_j;
  const float v = a.scale * sum;
  *o = a.accumulate ? *o + v : v;
}

hipError_t lora_tgrad(const LoraTGrad& a0, float* part, int64_t part_floats, hipStream_t s) {
  LoraTGrad a = a0;
  if (a.R <= 0 || a.njobs <= 0) return hipSuccess;
  if (a.njobs > 3 || a.r > 16) return hipErrorInvalidValue;
  // 32-bit byte offsets of the buffer loads
  if ((int64_t)TB * a.ldy * 4 >= BUF_OOB) return hipErrorInvalidValue;
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

hipError_t lora_mm(const LoraMM& a0, float* partial, int64_t partial_floats, hipStream_t s) {
  if (a0.R <= 0) return hipSuccess;
  if (a0.r > 16) return hipErrorInvalidValue;
  LoraMM a = a0;
  int ns, kc;
  split_of(a.R, a.K, &ns, &kc);
  if ((int64_t)ns * a.R * 16 > partial_floats || !partial) {  // no room: one pass over k
    ns = 1;
    kc = std::max(a.K, 1);
  }
  // extents of one block's buffer resources (every access outside them is
  // masked to BUF_OOB); the offsets are 32-bit
  const int64_t es = a.x_f32 ? 4 : 2;
  const int64_t xb = (a.trans ? (int64_t)(kc - 1) * a.ldx + 16 : 15 * a.ldx + kc) * es;
  const int64_t wb = ((int64_t)(kc - 1) * a.sk + (int64_t)std::max(a.r - 1, 0) * a.sj + 1) * 4;
  if (xb >= BUF_OOB || wb >= BUF_OOB) return hipErrorInvalidValue;
  a.xbytes = (uint32_t)xb;
  a.wbytes = (uint32_t)wb;
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
