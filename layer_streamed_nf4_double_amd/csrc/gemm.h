// Internal interface of the MFMA GEMM (see gemm.hip for the operand forms).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsn {

enum { A_BF16_K = 0, A_BF16_R = 1, A_F32_K = 2 };
enum { B_BF16_K = 0, B_BF16_R = 1, B_NF4_K = 2, B_NF4_R = 3 };
// C_SWIGLU (forward NF4 kernel only): B holds the fused gate|up rows
// [N = 2F, K]; the output is a = bf16(silu(gate) * up) [M, F] with row
// stride ldc, computed in the epilogue from the two accumulators
enum { C_F32 = 0, C_F32_ACC = 1, C_F32_RES = 2, C_BF16 = 3, C_SWIGLU = 4 };

struct GemmParams {
  int M = 0, N = 0, K = 0;
  const void* A = nullptr;
  int64_t lda = 0;
  const void* B = nullptr;  // bf16 matrix, or NF4 codes of W^T [rows, rowlen]
  int64_t ldb = 0;
  const float* absmax = nullptr;  // NF4 only: one float per 64 elements of W^T
  int64_t rowlen = 0;             // NF4 only: row length of W^T
  // batch index z = blockIdx.z split as (z / zdiv, z % zdiv); B uses the inner
  // index divided by grpB (grouped key/value heads)
  int zdiv = 1, grpB = 1;
  int64_t sA_o = 0, sA_i = 0, sB_o = 0, sB_i = 0, sC_o = 0, sC_i = 0;
  // the reduction runs over nseg segments of K each; segment s shifts A and B
  int nseg = 1;
  // causal attention products (M and K or M and N index the same sequence):
  // CAUSAL_SKIP_UPPER skips output tiles wholly above the diagonal (n > m),
  // which no consumer reads; CAUSAL_K_TO_ROW ends the reduction at the tile's
  // last row (A is zero for k > m); CAUSAL_K_FROM_ROW starts it at the tile's
  // first row, in every segment (A is zero for k < m)
  int causal = 0;
  int64_t sA_seg = 0, sB_seg = 0;
  // low-rank extension (bf16, k-contiguous, kext a multiple of 16)
  const uint16_t* Aext = nullptr;
  int64_t ldae = 0;
  const uint16_t* Bext = nullptr;
  int64_t ldbe = 0;
  int kext = 0;
  // output
  void* C = nullptr;
  int64_t ldc = 0;
  const float* R = nullptr;  // residual for C_F32_RES
  int64_t ldr = 0;
  float alpha = 1.f;
  int cmode = C_F32;
  // split-k scratch (fp32, split * split_stride(M, N)); without it the k range
  // is not split
  float* part = nullptr;
  int64_t part_floats = 0;
  int ksplit = 1;      // set by gemm()
  int64_t pstride = 0;  // floats from one split's partial sums to the next (set by gemm())
  // defer_reduce: a split launch leaves its partial sums (dense [M, N] rows,
  // buffer y at part + y pstride) for the consumer, which adds them in split
  // order; split_used (host, may be null) receives the split launched
  int defer_reduce = 0;
  int* split_used = nullptr;
  // optional timing events that record the main kernel's start and end (passed
  // to hipExtLaunchKernelGGL, so they add no dispatch of their own)
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  float levels[16] = {};  // NF4 code levels
};

// TILE_NF4F / TILE_NF4T: the 256 x 256 NF4 kernels of gemm_nf4f.hip (y = x W)
// and gemm_nf4t.hip (dx = dy W); TILE_BF16F: the 256 x 256 bf16 kernel of
// gemm_bf16.hip (C = A B^T, LM-head logits); TILE_BF16T: its C = A B
// counterpart (LM-head input gradient)
enum { CAUSAL_NONE = 0, CAUSAL_SKIP_UPPER = 1, CAUSAL_K_TO_ROW = 2, CAUSAL_K_FROM_ROW = 3 };

enum { TILE_256x128 = 0, TILE_128x128 = 1, TILE_64x64 = 2, TILE_NF4F = 3, TILE_NF4T = 4,
       TILE_BF16F = 5, TILE_BF16T = 6 };

struct GemmPlan {
  int tile = TILE_64x64;
  int split = 1;
};

// Floats from one split's partial-sum buffer to the next: M * N plus 4 KiB.
// The splits of a tile finish together and write their partial tiles at the
// same offsets of their buffers; buffers a multiple of the memory-channel
// interleave apart (M * N * 4 bytes often is) then send those writes to the
// same channels, which halves their rate on MI355X.
inline int64_t split_stride(int M, int N) { return (int64_t)M * N + 1024; }

hipError_t gemm(const GemmParams& p, int opa, int opb, int batch, hipStream_t s);
// the tile id gemm() launches for these operand forms
int gemm_tile(const GemmParams& p, int opa, int opb, int batch);
// the tile and split-k gemm() chooses for a problem
GemmPlan gemm_plan(int M, int N, int K, int nseg, int batch);
// fp32 scratch a split-k launch of this problem needs (0 when not split),
// for any operand forms
int64_t gemm_partial_floats(int M, int N, int K, int nseg, int batch);

// split-k reduction kernel (partial sums added in split order, then the epilogue)
__global__ void gemm_reduce_k(const GemmParams p);
// launches the reduction of p.ksplit partial sums (a vectorized form where the
// shapes allow it; both add in split order)
void gemm_reduce_launch(const GemmParams& p, hipStream_t s);

// forward NF4 kernel (gemm_nf4f.hip): y = x W with x bf16 [M, K] row-major and
// W^T NF4 [N, K]; used by gemm() whenever nf4f_eligible() holds
bool nf4f_eligible(const GemmParams& p, int batch);
// the k split of the 256 x 256 NF4 tile (both NF4 kernels)
int nf4f_split(int M, int N, int K);
// the forward kernel's column tiles per wave (nt = 2: 256 x 256 tile, 1:
// 256 x 128) and k split for a problem (gemm_partial_floats covers it)
struct Nf4fPlan {
  int nt, split;
};
Nf4fPlan nf4f_plan(int M, int N, int K);
hipError_t nf4f_launch(GemmParams p, hipStream_t s);
// whether the SwiGLU epilogue (cmode C_SWIGLU) takes this gate|up problem:
// the forward kernel takes it and its plan is the unsplit 256 x 256 tile,
// the one a plain fp32 launch of the same problem uses (so the gate and up
// values the epilogue sees are those a C_F32 launch would store)
bool nf4f_swiglu_ok(const GemmParams& p);

// input-gradient NF4 kernel (gemm_nf4t.hip): dx = dy W with dy bf16 [M, K]
// row-major and the same W^T NF4 record [K, N] (operand form B_NF4_R); used by
// gemm() whenever nf4t_eligible() holds; splits the k range like nf4f
bool nf4t_eligible(const GemmParams& p, int batch);
hipError_t nf4t_launch(GemmParams p, hipStream_t s);

// bf16 kernel (gemm_bf16.hip): C = A B^T with A [M, K] and B [N, K] bf16,
// both k-contiguous (operand forms A_BF16_K, B_BF16_K); used by gemm()
// whenever bf16f_eligible() holds; splits the k range like nf4f
bool bf16f_eligible(const GemmParams& p, int batch);
hipError_t bf16f_launch(GemmParams p, hipStream_t s);
// ... and C = A B with B [K, N] bf16, N contiguous (operand form B_BF16_R)
bool bf16t_eligible(const GemmParams& p, int batch);
hipError_t bf16t_launch(GemmParams p, hipStream_t s);

}  // namespace lsn
