// bf16 GEMMs of the LM head for full 64-deep K slices, built like the NF4
// kernels (gemm_nf4f.hip, gemm_nf4t.hip) with the weight tile loaded as bf16
// instead of decoded:
//
//   bf16f_kernel  C[m, n] (op)= sum_k A[m, k] * B[n, k]    (B [N, K]: logits =
//                 hidden states times the embedding rows of a vocabulary chunk)
//   bf16t_kernel  C[m, n] (op)= sum_k A[m, k] * B[k, n]    (B [K, N]: the input
//                 gradient dlogits times those embedding rows)
//
// Work split.  A workgroup of four waves owns a 256 x 256 output tile; wave w
// owns all 256 rows and the 64 columns n0 + 64w .. +63 (8 x 2 MFMA tiles of
// 32 x 32, 256 fp32 accumulators per lane).  The B rows of a wave are used by
// that wave only, so each wave direct-loads its own 64 x 64 B slice into LDS
// it alone reads (no barrier); the A slice [256 x 64] is shared through LDS.
//
// Memory pipeline (both kernels): A in three LDS stages, B in two (160 KiB in
// all).  Both arrive by direct loads
// (global_load_lds_dwordx4), XOR-swizzled by row so that the fragment reads
// are free of bank conflicts.  In k-step 3 of slice t, after the slice's
// barrier, a wave issues B of slice t + 2 (its stage was last read in k-step
// 2) and then its share of A of slice t + 3.  Before the next barrier it
// waits until only that A share may still be in flight.
//
// Determinism: every output element is reduced by one lane in a fixed order.
#include "common.h"
#include <hip/hip_ext.h>

#include "gemm.h"
#include "nf4_direct.h"
#include <algorithm>
#include <type_traits>

namespace lsn {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int A_ST = 3, B_ST = 2;        // LDS stages
constexpr int STAGE = BM * BK * 2;       // 32 KiB (A slice; B slices of four waves)

}  // namespace

// MODE: the output form (C_F32, C_F32_ACC, C_F32_RES, C_BF16), or -1 for the
// raw split-k partial sums.
template <int MODE>
__global__ __launch_bounds__(256) void bf16f_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA[A_ST][STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB[B_ST][STAGE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lr = lane & 31, hh = lane >> 5;

  // ---- tile coordinates and k split (XCD-aware, split-major) ----
  const int mt = (p.M + BM - 1) / BM;
  const WorkUnit wu = xcd_unit();
  const int id = wu.tile, ks = wu.split;
  const int m0 = (id % mt) * BM, n0 = (id / mt) * BN;

  // ---- direct-load byte offsets of this lane (slice 0) ----
  // A: load i of wave w fills stage rows (8w + i) * 8 .. +7 (shared);
  // B: load i of wave w fills rows 8i .. +7 of the wave's own 64-row block.
  // lane -> row + lane / 8, physical chunk lane % 8 (logical chunk c ^ swz)
  uint32_t offA[8], offB[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (w * 8 + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    offA[i] = (uint32_t)(((int64_t)min(m0 + r, p.M - 1) * p.lda + c * 8) * 2);
    const int rb = i * 8 + (lane >> 3);
    const int cb = (lane & 7) ^ swz(rb);
    offB[i] = (uint32_t)(((int64_t)min(n0 + w * 64 + rb, p.N - 1) * p.ldb + cb * 8) * 2);
  }
  // the same offsets for one M0 per group, loads at instruction offsets
  // 1024 i - 4096; never negative (load i covers rows >= 8 i of a matrix whose
  // rows are at least 128 bytes long)
  uint32_t offA_o[8], offB_o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    offA_o[i] = offA[i] + 4096u - 1024u * i;
    offB_o[i] = offB[i] + 4096u - 1024u * i;
  }

  const uint8_t* gA = reinterpret_cast<const uint8_t*>(p.A);
  const uint8_t* gB = reinterpret_cast<const uint8_t*>(p.B);

  // split-k: split ks takes slices [it0, it1)
  const int nkt = p.K / BK;
  const int kper = (nkt + p.ksplit - 1) / p.ksplit;
  const int it0 = min(nkt, ks * kper), it1 = min(nkt, it0 + kper);

  auto issue_a = [&](int it, int st) {
    const uint8_t* a = gA + it * (BK * 2);
    const uint32_t la = lds_addr(sA[st]) + w * 8 * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(a, offA[i], la + i * 1024);
  };
  auto issue_b = [&](int it, int st) {
    const uint8_t* bp = gB + it * (BK * 2);
    const uint32_t lb = lds_addr(sB[st]) + w * 8 * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(bp, offB[i], lb + i * 1024);
  };

  // fragment of row tile i (A) or column tile j of this wave (B), k-step kk:
  // row 32 * tile + lr, logical chunk 4*hh + kk -> physical (4*hh ^ swz(lr)) ^ kk
  const int sa0 = lr * 128 + (((4 * hh) ^ swz(lr)) * 16);
  const int sb0 = w * 8 * 1024 + sa0;

  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  bf16x8 af[2][8];  // A fragments, double buffered over k-steps
  bf16x8 bq[2][2];  // B fragments [kk & 1][column tile]

  // One k-step as 16 MFMA slots (row tile s/2, column tile s%2), with the
  // next k-step's A fragments (slots 0-7) and B fragments (slots 8, 9) read
  // between them (sched_barrier after every slot).  extra(s) adds per-slot
  // work (the direct loads of the last k-step).
  auto kstep = [&](auto kk_, const uint8_t* an, const uint8_t* bn, auto extra) {
    constexpr int F = decltype(kk_)::value & 1;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      acc[s >> 1][s & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          bq[F][s & 1], af[F][s >> 1], acc[s >> 1][s & 1], 0, 0, 0);
      if (s < 8) af[F ^ 1][s] = *reinterpret_cast<const bf16x8*>(an + s * 4096);
      if (s == 8 || s == 9) bq[F ^ 1][s - 8] = *reinterpret_cast<const bf16x8*>(bn + (s - 8) * 4096);
      extra(s);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto none = [](int) {};

  if (it1 > it0) {
    // prologue: A of slices it0 .. it0+2 into A stages 0 .. 2, B of slices
    // it0, it0+1 into B stages 0, 1 (clamped), in the order the loop expects
    issue_b(it0, 0);
    issue_a(it0, 0);
    issue_b(min(it0 + 1, it1 - 1), 1);
    issue_a(min(it0 + 1, it1 - 1), 1);
    issue_a(min(it0 + 2, it1 - 1), 2);
    LSN_WAIT_VM(16);  // slice it0 (and B of it0 + 1) landed
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) af[0][i] = *reinterpret_cast<const bf16x8*>(sA[0] + sa0 + i * 4096);
#pragma unroll
    for (int j = 0; j < 2; ++j) bq[0][j] = *reinterpret_cast<const bf16x8*>(sB[0] + sb0 + j * 4096);
    // Slice t (u = t - it0): A in stage u % 3, B in stage u % 2.  Before the
    // barrier of slice t this wave waits for its loads of A(t + 1) and
    // B(t + 1) (only its A share of t + 2 may be in flight); the barrier makes
    // A(t + 1) visible and frees A stage u % 3, and k-step 3 refills B stage
    // u % 2 with B(t + 2) and A stage u % 3 with A(t + 3).
    int st = 0, sb = 0;
    for (int t = it0; t < it1; ++t) {
      const int st1 = st == A_ST - 1 ? 0 : st + 1, sb1 = sb ^ 1;
      kstep(std::integral_constant<int, 0>{}, sA[st] + (sa0 ^ 16), sB[sb] + (sb0 ^ 16), none);
      kstep(std::integral_constant<int, 1>{}, sA[st] + (sa0 ^ 32), sB[sb] + (sb0 ^ 32), none);
      kstep(std::integral_constant<int, 2>{}, sA[st] + (sa0 ^ 48), sB[sb] + (sb0 ^ 48), none);
      LSN_WAIT_VM(8);
      __syncthreads();  // (its fence waits lgkmcnt(0): this wave's reads of stage st / sb are done)
      const uint8_t* a_next = gA + min(t + 3, it1 - 1) * (BK * 2);
      const uint8_t* b_next = gB + min(t + 2, it1 - 1) * (BK * 2);
      const uint32_t la = lds_addr(sA[st]) + w * 8 * 1024;
      const uint32_t lb = lds_addr(sB[sb]) + w * 8 * 1024;
      kstep(std::integral_constant<int, 3>{}, sA[st1] + sa0, sB[sb1] + sb0, [&](int s) {
        // one M0 per group; the loads address relative to it
        if (s == 0) {
          set_m0(lb + 4096);
          dma16_at<-4096>(b_next, offB_o[0]);
        }
        if (s == 1) dma16_at<-3072>(b_next, offB_o[1]);
        if (s == 2) dma16_at<-2048>(b_next, offB_o[2]);
        if (s == 3) dma16_at<-1024>(b_next, offB_o[3]);
        if (s == 4) dma16_at<0>(b_next, offB_o[4]);
        if (s == 5) dma16_at<1024>(b_next, offB_o[5]);
        if (s == 6) dma16_at<2048>(b_next, offB_o[6]);
        if (s == 7) dma16_at<3072>(b_next, offB_o[7]);
        if (s == 8) {
          set_m0(la + 4096);
          dma16_at<-4096>(a_next, offA_o[0]);
        }
        if (s == 9) dma16_at<-3072>(a_next, offA_o[1]);
        if (s == 10) dma16_at<-2048>(a_next, offA_o[2]);
        if (s == 11) dma16_at<-1024>(a_next, offA_o[3]);
        if (s == 12) dma16_at<0>(a_next, offA_o[4]);
        if (s == 13) dma16_at<1024>(a_next, offA_o[5]);
        if (s == 14) dma16_at<2048>(a_next, offA_o[6]);
        if (s == 15) dma16_at<3072>(a_next, offA_o[7]);
      });
      st = st1;
      sb = sb1;
    }
    LSN_WAIT_VM(0);  // no direct load may still be writing LDS when the waves exit
  }

  // ---- epilogue (as in the forward NF4 kernel) ----
  // Tile (i, j) holds the transpose: lane (lr, hh) has output row
  // m = m0 + 32i + lr and the columns n = n0 + 64w + 32j + 8g + 4hh + t in
  // acc[i][j][4g + t], four consecutive columns per 16-byte store.
  auto epilogue = [&](auto full_) {
    constexpr bool FULL = decltype(full_)::value;
    constexpr bool LOADS = MODE == C_F32_ACC || MODE == C_F32_RES;
    float* const out = MODE < 0 ? p.part + ks * p.pstride : reinterpret_cast<float*>(p.C);
    const int64_t ld = MODE < 0 ? (int64_t)p.N : p.ldc;
    const float* const src = MODE == C_F32_RES ? p.R : out;
    const int64_t lds = MODE == C_F32_RES ? p.ldr : ld;
    const int nl = n0 + w * 64 + hh * 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = m0 + i * 32 + lr;
      if (!FULL && m >= p.M) continue;
      float* __restrict__ orow = out + (int64_t)m * ld + nl;
      uint16_t* __restrict__ brow = reinterpret_cast<uint16_t*>(p.C) + (int64_t)m * ld + nl;
      const float* __restrict__ srow = src + (int64_t)m * lds + nl;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = j * 32 + g * 8;
          if (!FULL && nl + c >= p.N) continue;
          f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                     acc[i][j][4 * g + 3]};
          if constexpr (LOADS) v += *reinterpret_cast<const f32x4*>(srow + c);
          if constexpr (MODE == C_BF16) {
            u32x2 b2 = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            *reinterpret_cast<u32x2*>(brow + c) = b2;
          } else {
            *reinterpret_cast<f32x4*>(orow + c) = v;
          }
        }
    }
  };
  if (m0 + BM <= p.M && n0 + BN <= p.N) epilogue(std::true_type{});
  else epilogue(std::false_type{});
}

// bf16t_kernel: B is [K, N] with N contiguous (the embedding rows of the
// chunk).  An MFMA fragment needs eight consecutive k of one column, while a
// 32-bit word of a B row holds two adjacent columns; so, as in the NF4 input
// gradient kernel, lane l of a column-tile pair takes columns 2l (tile 0) and
// 2l + 1 (tile 1) of the wave's 64: one 4-byte LDS read per k row feeds both
// tiles, and byte permutes split the eight words into the two fragments.
// A wave's B block holds its 64 k rows x 128 bytes; the two lane halves read
// rows k and k + 32 together, so rows 32..63 are stored with adjacent rows
// swapped, which puts every such pair in different halves of a bank window.
template <int MODE>
__global__ __launch_bounds__(256) void bf16t_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA[A_ST][STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB[B_ST][STAGE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lr = lane & 31, hh = lane >> 5;

  const int mt = (p.M + BM - 1) / BM;
  const WorkUnit wu = xcd_unit();
  const int id = wu.tile, ks = wu.split;
  const int m0 = (id % mt) * BM, n0 = (id / mt) * BN;
  const int nw = n0 + 64 * w;              // this wave's first column
  const int nwl = min(nw, p.N - 64);       // the same, kept inside the matrix for loads

  // A: as in bf16f_kernel.  B: load i of wave w fills row slots 8i .. +7 of
  // the wave's block (lane -> slot 8i + lane / 8, 16-byte chunk lane % 8);
  // slot s holds k row s below 32 and row s ^ 1 from 32 on.
  uint32_t offA[8], offB[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (w * 8 + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    offA[i] = (uint32_t)(((int64_t)min(m0 + r, p.M - 1) * p.lda + c * 8) * 2);
    const int slot = i * 8 + (lane >> 3);
    const int krow = slot < 32 ? slot : (slot ^ 1);
    offB[i] = (uint32_t)(((int64_t)krow * p.ldb + nwl) * 2 + (lane & 7) * 16);
  }
  uint32_t offA_o[8], offB_o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    offA_o[i] = offA[i] + 4096u - 1024u * i;
    offB_o[i] = offB[i] + 4096u - 1024u * i;  // load i covers k rows >= 8 i of 128+ bytes
  }

  const uint8_t* gA = reinterpret_cast<const uint8_t*>(p.A);
  const uint8_t* gB = reinterpret_cast<const uint8_t*>(p.B);
  const int64_t bstep = (int64_t)BK * p.ldb * 2;  // bytes of B per slice

  const int nkt = p.K / BK;
  const int kper = (nkt + p.ksplit - 1) / p.ksplit;
  const int it0 = min(nkt, ks * kper), it1 = min(nkt, it0 + kper);

  auto issue_a = [&](int it, int st) {
    const uint8_t* a = gA + it * (BK * 2);
    const uint32_t la = lds_addr(sA[st]) + w * 8 * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(a, offA[i], la + i * 1024);
  };
  auto issue_b = [&](int it, int st) {
    const uint8_t* bp = gB + it * bstep;
    const uint32_t lb = lds_addr(sB[st]) + w * 8 * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(bp, offB[i], lb + i * 1024);
  };

  const int sa0 = lr * 128 + (((4 * hh) ^ swz(lr)) * 16);
  // B word of column pair lr in k row 32*hh + 8*kk + e: slot 8kk + e (hh = 0)
  // or 32 + ((8kk + e) ^ 1) (hh = 1); separate bases for even and odd e
  const int sbe = w * 8 * 1024 + hh * (4096 + 128) + 4 * lr;
  const int sbo = w * 8 * 1024 + hh * (4096 - 128) + 4 * lr;

  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  bf16x8 af[2][8];
  bf16x8 bq[2][2];
  uint32_t bw[8];  // B words of the next k-step

  // the eight words (k rows, each two columns) -> the two column fragments
  auto split = [&](int F) {
    u32x4 lo, hi;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lo[q] = __builtin_amdgcn_perm(bw[2 * q + 1], bw[2 * q], 0x05040100u);  // low halves
      hi[q] = __builtin_amdgcn_perm(bw[2 * q + 1], bw[2 * q], 0x07060302u);  // high halves
    }
    bq[F][0] = __builtin_bit_cast(bf16x8, lo);
    bq[F][1] = __builtin_bit_cast(bf16x8, hi);
  };
  auto read_words = [&](const uint8_t* bs, int kk, int e) {
    bw[e] = *reinterpret_cast<const uint32_t*>(bs + ((e & 1) ? sbo : sbe) + (8 * kk + e) * 128);
  };

  // one k-step: 16 MFMA slots; the next k-step's A fragments (slots 0-7) and
  // B words (slots 0-7), then the split into fragments (slot 12)
  auto kstep = [&](auto kk_, const uint8_t* an, const uint8_t* bs, int kn, auto extra) {
    constexpr int F = decltype(kk_)::value & 1;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      acc[s >> 1][s & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          bq[F][s & 1], af[F][s >> 1], acc[s >> 1][s & 1], 0, 0, 0);
      if (s < 8) {
        af[F ^ 1][s] = *reinterpret_cast<const bf16x8*>(an + s * 4096);
        read_words(bs, kn, s);
      }
      if (s == 12) split(F ^ 1);
      extra(s);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto none = [](int) {};

  if (it1 > it0) {
    issue_b(it0, 0);
    issue_a(it0, 0);
    issue_b(min(it0 + 1, it1 - 1), 1);
    issue_a(min(it0 + 1, it1 - 1), 1);
    issue_a(min(it0 + 2, it1 - 1), 2);
    LSN_WAIT_VM(16);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) af[0][i] = *reinterpret_cast<const bf16x8*>(sA[0] + sa0 + i * 4096);
#pragma unroll
    for (int e = 0; e < 8; ++e) read_words(sB[0], 0, e);
    split(0);
    // as in bf16f_kernel: A(t) in stage u % 3, B(t) in stage u % 2
    int st = 0, sb = 0;
    for (int t = it0; t < it1; ++t) {
      const int st1 = st == A_ST - 1 ? 0 : st + 1, sb1 = sb ^ 1;
      kstep(std::integral_constant<int, 0>{}, sA[st] + (sa0 ^ 16), sB[sb], 1, none);
      kstep(std::integral_constant<int, 1>{}, sA[st] + (sa0 ^ 32), sB[sb], 2, none);
      kstep(std::integral_constant<int, 2>{}, sA[st] + (sa0 ^ 48), sB[sb], 3, none);
      LSN_WAIT_VM(8);
      __syncthreads();
      const uint8_t* a_next = gA + min(t + 3, it1 - 1) * (BK * 2);
      const uint8_t* b_next = gB + min(t + 2, it1 - 1) * bstep;
      const uint32_t la = lds_addr(sA[st]) + w * 8 * 1024;
      const uint32_t lb = lds_addr(sB[sb]) + w * 8 * 1024;
      kstep(std::integral_constant<int, 3>{}, sA[st1] + sa0, sB[sb1], 0, [&](int s) {
        if (s == 0) {
          set_m0(lb + 4096);
          dma16_at<-4096>(b_next, offB_o[0]);
        }
        if (s == 1) dma16_at<-3072>(b_next, offB_o[1]);
        if (s == 2) dma16_at<-2048>(b_next, offB_o[2]);
        if (s == 3) dma16_at<-1024>(b_next, offB_o[3]);
        if (s == 4) dma16_at<0>(b_next, offB_o[4]);
        if (s == 5) dma16_at<1024>(b_next, offB_o[5]);
        if (s == 6) dma16_at<2048>(b_next, offB_o[6]);
        if (s == 7) dma16_at<3072>(b_next, offB_o[7]);
        if (s == 8) {
          set_m0(la + 4096);
          dma16_at<-4096>(a_next, offA_o[0]);
        }
        if (s == 9) dma16_at<-3072>(a_next, offA_o[1]);
        if (s == 10) dma16_at<-2048>(a_next, offA_o[2]);
        if (s == 11) dma16_at<-1024>(a_next, offA_o[3]);
        if (s == 12) dma16_at<0>(a_next, offA_o[4]);
        if (s == 13) dma16_at<1024>(a_next, offA_o[5]);
        if (s == 14) dma16_at<2048>(a_next, offA_o[6]);
        if (s == 15) dma16_at<3072>(a_next, offA_o[7]);
      });
      st = st1;
      sb = sb1;
    }
    LSN_WAIT_VM(0);
  }

  // ---- epilogue (as in the NF4 input-gradient kernel) ----
  // lane (lr, hh): row m = m0 + 32i + lr, column nw + 16g + 8hh + 2t + j in
  // acc[i][j][4g + t]; eight consecutive columns per (i, g).  N is a multiple
  // of 64, so a wave's columns are all inside the matrix or all outside.
  auto epilogue = [&](auto full_) {
    constexpr bool FULL = decltype(full_)::value;
    constexpr bool LOADS = MODE == C_F32_ACC || MODE == C_F32_RES;
    if (!FULL && nw >= p.N) return;
    float* const out = MODE < 0 ? p.part + ks * p.pstride : reinterpret_cast<float*>(p.C);
    const int64_t ld = MODE < 0 ? (int64_t)p.N : p.ldc;
    const float* const src = MODE == C_F32_RES ? p.R : out;
    const int64_t lds = MODE == C_F32_RES ? p.ldr : ld;
    const int nl = nw + hh * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = m0 + i * 32 + lr;
      if (!FULL && m >= p.M) continue;
      float* __restrict__ orow = out + (int64_t)m * ld + nl;
      uint16_t* __restrict__ brow = reinterpret_cast<uint16_t*>(p.C) + (int64_t)m * ld + nl;
      const float* __restrict__ srow = src + (int64_t)m * lds + nl;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = g * 16;
        f32x4 v0 = {acc[i][0][4 * g], acc[i][1][4 * g], acc[i][0][4 * g + 1], acc[i][1][4 * g + 1]};
        f32x4 v1 = {acc[i][0][4 * g + 2], acc[i][1][4 * g + 2], acc[i][0][4 * g + 3],
                    acc[i][1][4 * g + 3]};
        if constexpr (LOADS) {
          v0 += *reinterpret_cast<const f32x4*>(srow + c);
          v1 += *reinterpret_cast<const f32x4*>(srow + c + 4);
        }
        if constexpr (MODE == C_BF16) {
          u32x4 b4 = {pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]),
                      pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
          *reinterpret_cast<u32x4*>(brow + c) = b4;
        } else {
          *reinterpret_cast<f32x4*>(orow + c) = v0;
          *reinterpret_cast<f32x4*>(orow + c + 4) = v1;
        }
      }
    }
  };
  if (m0 + BM <= p.M && n0 + BN <= p.N) epilogue(std::true_type{});
  else epilogue(std::false_type{});
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static bool aligned_to(const void* q, uintptr_t a) { return ((uintptr_t)q & (a - 1)) == 0; }

bool bf16f_eligible(const GemmParams& p, int batch) {
  if (batch != 1 || p.nseg != 1 || p.zdiv != 1 || p.alpha != 1.f || p.kext != 0 || p.causal)
    return false;
  if (p.M < BM || p.N < 64 || p.K % BK != 0) return false;
  if (p.lda % 8 != 0 || p.ldb % 8 != 0 || p.lda < 64 || p.ldb < 64 || !aligned_to(p.A, 16) ||
      !aligned_to(p.B, 16))
    return false;
  if (p.N % 4 != 0 || p.ldc % 4 != 0 || !aligned_to(p.C, 16) || !aligned_to(p.part, 16)) return false;
  if (p.cmode == C_F32_RES && (p.ldr % 4 != 0 || !aligned_to(p.R, 16))) return false;
  const int64_t lim = (int64_t)1 << 31;
  return (int64_t)p.M * p.lda * 2 < lim && (int64_t)p.N * p.ldb * 2 < lim;
}

bool bf16t_eligible(const GemmParams& p, int batch) {
  if (batch != 1 || p.nseg != 1 || p.zdiv != 1 || p.alpha != 1.f || p.kext != 0 || p.causal)
    return false;
  if (p.M < BM || p.N < 64 || p.N % 64 != 0 || p.K % BK != 0) return false;
  if (p.lda % 8 != 0 || p.lda < 64 || p.ldb % 8 != 0 || p.ldb < p.N || !aligned_to(p.A, 16) ||
      !aligned_to(p.B, 16))
    return false;
  if (p.ldc % 8 != 0 || !aligned_to(p.C, 16) || !aligned_to(p.part, 16)) return false;
  if (p.cmode == C_F32_RES && (p.ldr % 4 != 0 || !aligned_to(p.R, 16))) return false;
  const int64_t lim = (int64_t)1 << 31;
  return (int64_t)p.M * p.lda * 2 < lim && (int64_t)BK * p.ldb * 2 < lim;
}

hipError_t bf16t_launch(GemmParams p, hipStream_t s) {
  p.ksplit = nf4f_split(p.M, p.N, p.K);
  p.pstride = split_stride(p.M, p.N);
  if (p.ksplit > 1 && (!p.part || p.part_floats < p.ksplit * p.pstride)) p.ksplit = 1;
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const dim3 grid(tiles, p.ksplit, 1);
  if (p.ksplit > 1)
    hipExtLaunchKernelGGL(bf16t_kernel<-1>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32)
    hipExtLaunchKernelGGL(bf16t_kernel<C_F32>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32_ACC)
    hipExtLaunchKernelGGL(bf16t_kernel<C_F32_ACC>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32_RES)
    hipExtLaunchKernelGGL(bf16t_kernel<C_F32_RES>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else
    hipExtLaunchKernelGGL(bf16t_kernel<C_BF16>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  if (p.split_used) *p.split_used = p.ksplit;
  if (p.ksplit > 1 && !p.defer_reduce) gemm_reduce_launch(p, s);
  return hipGetLastError();
}

hipError_t bf16f_launch(GemmParams p, hipStream_t s) {
  p.ksplit = nf4f_split(p.M, p.N, p.K);
  p.pstride = split_stride(p.M, p.N);
  if (p.ksplit > 1 && (!p.part || p.part_floats < p.ksplit * p.pstride)) p.ksplit = 1;
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const dim3 grid(tiles, p.ksplit, 1);
  if (p.ksplit > 1)
    hipExtLaunchKernelGGL(bf16f_kernel<-1>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32)
    hipExtLaunchKernelGGL(bf16f_kernel<C_F32>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32_ACC)
    hipExtLaunchKernelGGL(bf16f_kernel<C_F32_ACC>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32_RES)
    hipExtLaunchKernelGGL(bf16f_kernel<C_F32_RES>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else
    hipExtLaunchKernelGGL(bf16f_kernel<C_BF16>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  if (p.split_used) *p.split_used = p.ksplit;
  if (p.ksplit > 1 && !p.defer_reduce) gemm_reduce_launch(p, s);
  return hipGetLastError();
}

}  // namespace lsn
