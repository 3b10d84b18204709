// Forward NF4 projection y = x W for full 64-deep K slices, built around the
// matrix cores of one CDNA4 compute unit.
//
//   C[m, n] (op)= sum_k x[m, k] * bf16(level[code(n, k)] * absmax(n, k))
//                 (+ the low-rank extension of gemm.hip)
//
// The weight is the NF4 record's W^T [N, K] (codes two per byte, even element
// in the low nibble, one fp32 absmax per 64 consecutive elements of a row),
// so every 64-deep K slice of a row is exactly one absmax block.
//
// Work split.  A workgroup of four waves (one per SIMD) owns a 256 x 256
// output tile; wave w owns all 256 rows and the 64 columns n0 + 64w .. +63,
// i.e. 8 x 2 tiles of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per
// lane).  Because the waves split only the N dimension, each weight element
// of the tile is dequantized exactly once per workgroup, directly into the
// B-fragment registers of the wave that uses it; the dequantized weight never
// passes through LDS.  Only the activation slice [256 x 64] is shared through
// LDS, so LDS read traffic per MFMA is half that of a 64 x 64 wave tile that
// reads both operands from LDS.
//
// K order inside a slice.  An MFMA sums over 16 k; which 16 of the slice's 64
// it takes is free as long as both operands agree.  Lane half h (lane / 32)
// takes k = 32h + 8kk .. +7 in k-step kk, so each lane's weight codes for a
// whole slice are 16 contiguous bytes (one load) and its activation chunks
// are the 16-byte chunks 4h + kk of its rows.
//
// Memory pipeline (one iteration = one slice).  Activations, codes and
// absmax go global -> LDS with direct loads (global_load_lds_dwordx4 /
// _dword), three slices ahead, into three LDS stages; a slice's activation
// chunks are XOR-swizzled by row so the fragment reads (ds_read_b128) are
// free of bank conflicts.  The direct loads are issued from inline asm: the
// compiler does not see them, so it cannot order every later LDS read behind
// them; the kernel itself waits for its own loads (vmcnt) and then meets the
// other waves at one barrier per slice, placed before the last k-step so the
// next slice's first fragments load while the last MFMAs run.  Weight codes
// are dequantized just in time, one k-step ahead of their MFMAs: each code
// byte indexes a 256-entry LDS table holding the levels of its two nibbles.
//
// Determinism: every output element is reduced by one lane in a fixed order
// (split-k partial sums are added in split order by gemm_reduce_launch).
#include "common.h"
#include <hip/hip_ext.h>

#include "gemm.h"
#include "nf4_direct.h"
#include <algorithm>
#include <type_traits>

namespace lsn {

namespace {

constexpr int FM = 256, FN = 256, FK = 64;
constexpr int NST = 3;                 // LDS stages
constexpr int A_STAGE = FM * FK * 2;   // 32 KiB of activations (bf16)
constexpr int C_STAGE = FN * FK / 2;   // 8 KiB of codes
constexpr int GROUP = 8 + 2 + 1;       // direct loads per wave per slice

// Eight NF4 codes (one 32-bit word; element 2p in the low nibble of byte p)
// to eight bf16 products level * absmax, each rounded once.
template <typename Pair>
LSN_DEV bf16x8 dequant8(uint32_t q, float a, Pair pair) {
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float2 l = pair(pair_off(q, p));
    r[p] = pack_bf16x2(l.x * a, l.y * a);
  }
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace

// MODE: the output form (C_F32, C_F32_ACC, C_F32_RES, C_BF16), or -1 for the
// raw split-k partial sums; one instantiation per form keeps the epilogue a
// single straight-line path per tile kind.
template <int MODE>
__global__ __launch_bounds__(256) void nf4f_kernel(const GemmParams p) {
  // the level-pair table first: its LDS address fits the 16-bit ds_read offset
  __shared__ __attribute__((aligned(64))) float2 sPair[256];
  __shared__ __attribute__((aligned(1024))) uint8_t sA[NST][A_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sC[NST][C_STAGE];
  __shared__ __attribute__((aligned(1024))) float sM[NST][FN];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lr = lane & 31, hh = lane >> 5;

  // ---- tile coordinates (XCD-aware: consecutive ids land on one XCD) ----
  const int mt = (p.M + FM - 1) / FM;
  const int nblk = gridDim.x, b = blockIdx.x;
  const int per = nblk / 8, rem = nblk % 8, x = b % 8;
  const int id = x * per + min(x, rem) + b / 8;
  const int m0 = (id % mt) * FM, n0 = (id / mt) * FN;

  // entry b: the levels of code byte b (low nibble: even element, high
  // nibble: odd element); one 8-byte read dequantizes two elements
  sPair[threadIdx.x] = make_float2(p.levels[threadIdx.x & 15], p.levels[threadIdx.x >> 4]);
  auto pair = [&](uint32_t b8) {  // b8 = 8 * code byte
    return *reinterpret_cast<const float2*>(reinterpret_cast<const char*>(sPair) + b8);
  };

  // ---- direct-load byte offsets of this lane (slice 0) ----
  // activations: load i of wave w fills stage rows (8w + i) * 8 .. +7;
  // lane -> row + lane / 8, physical chunk lane % 8
  uint32_t offA[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (w * 8 + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    const int row = min(m0 + r, p.M - 1);
    offA[i] = (uint32_t)(((int64_t)row * p.lda + c * 8) * 2);
  }
  // codes: load i of wave w fills weight rows (2w + i) * 32 .. +31 (32 B
  // each); lane -> row + lane / 2, physical half lane % 2
  uint32_t offC[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (w * 2 + i) * 32 + (lane >> 1);
    const int h = (lane & 1) ^ ((r >> 3) & 1);
    const int row = min(n0 + r, p.N - 1);
    offC[i] = (uint32_t)((int64_t)row * (p.K / 2) + h * 16);
  }
  // the same offsets for loads at instruction offset 1024 i - 4096 from one
  // M0 (activation load i) and at 1024 i (code load i); never negative,
  // since load i covers rows >= 8 i (activations) or >= 32 i (codes)
  uint32_t offA_o[8], offC_o[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) offA_o[i] = offA[i] + 4096u - 1024u * i;
  offC_o[0] = offC[0];
  offC_o[1] = offC[1] - 1024u;
  // absmax: wave w fills rows 64w .. +63, lane -> row 64w + lane
  const uint32_t offM =
      (uint32_t)((int64_t)min(n0 + w * 64 + lane, p.N - 1) * (p.K / FK) * 4);

  const uint8_t* gA = reinterpret_cast<const uint8_t*>(p.A);
  const uint8_t* gC = reinterpret_cast<const uint8_t*>(p.B);
  const uint8_t* gM = reinterpret_cast<const uint8_t*>(p.absmax);

  // split-k: blockIdx.y takes slices [it0, it1)
  const int nkt = p.K / FK;
  const int kper = (nkt + p.ksplit - 1) / p.ksplit;
  const int it0 = min(nkt, (int)blockIdx.y * kper), it1 = min(nkt, it0 + kper);

  // the GROUP direct loads of slice it into LDS stage st
  auto issue = [&](int it, int st) {
    const uint8_t* a = gA + it * (FK * 2);
    const uint32_t la = lds_addr(sA[st]) + w * 8 * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(a, offA[i], la + i * 1024);
    const uint8_t* c = gC + it * (FK / 2);
    const uint32_t lc = lds_addr(sC[st]) + w * 2 * 1024;
    dma16(c, offC[0], lc);
    dma16(c, offC[1], lc + 1024);
    dma4(gM + it * 4, offM, lds_addr(&sM[st][w * 64]));
  };

  // ---- per-lane LDS read offsets ----
  // activation fragment of row tile i, k-step kk: row i*32 + lr, logical chunk
  // 4*hh + kk -> physical (4*hh ^ swz(lr)) ^ kk (kk only flips the low bits)
  const int sa0 = lr * 128 + (((4 * hh) ^ swz(lr)) * 16);
  // codes of column tile j: row 64w + 32j + lr, logical half hh
  const int sc0 = (w * 64 + lr) * 32 + ((hh ^ ((lr >> 3) & 1)) * 16);
  const int sm0 = w * 64 + lr;

  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  bf16x8 af[2][8];  // activation fragments, double buffered over k-steps
  bf16x8 bq[2][2];  // weight fragments [kk & 1][j]
  u32x4 cq[2], cqn[2];  // codes of this slice and of the next one (per column tile)
  float ca[2], can[2];

  auto read_codes = [&](u32x4 (&q)[2], float (&a)[2], int st) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      q[j] = *reinterpret_cast<const u32x4*>(sC[st] + sc0 + j * 1024);
      a[j] = sM[st][sm0 + j * 32];
    }
  };

  // One k-step as 16 MFMA slots (row tile s/2, column tile s%2).  Between
  // them, in a fixed order (sched_barrier after every slot): the next
  // k-step's eight activation fragments and the eight level-pair reads of
  // its two weight tiles (slots 0-7), then the products and bf16 packing
  // (slots 8-15, when the reads have long returned).
  // extra(s) adds per-slot work (the direct loads of the last k-step).
  auto kstep = [&](auto kk_, const uint8_t* an, const u32x4 (&q)[2], const float (&a)[2],
                   int kn, auto extra) {
    constexpr int F = decltype(kk_)::value & 1;
    float lvv[2][8];
    u32x4 r[2];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      acc[s >> 1][s & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          bq[F][s & 1], af[F][s >> 1], acc[s >> 1][s & 1], 0, 0, 0);
      if (s < 8) af[F ^ 1][s] = *reinterpret_cast<const bf16x8*>(an + s * 4096);
      if (s < 8) {  // level pair ph of tile jt (byte ph of the code word)
        const int jt = s >> 2, ph = s & 3;
        const float2 l = pair(pair_off(q[jt][kn], ph));
        lvv[jt][2 * ph] = l.x;
        lvv[jt][2 * ph + 1] = l.y;
      } else {
        const int jt = (s - 8) >> 2, pp = (s - 8) & 3;
        r[jt][pp] = pack_bf16x2(lvv[jt][2 * pp] * a[jt], lvv[jt][2 * pp + 1] * a[jt]);
        if (pp == 3) bq[F ^ 1][jt] = __builtin_bit_cast(bf16x8, r[jt]);
      }
      extra(s);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto none = [](int) {};

  if (it1 > it0) {
    // prologue: slices it0 .. it0+2 (clamped) into stages 0 .. 2
    issue(it0, 0);
    issue(min(it0 + 1, it1 - 1), 1);
    issue(min(it0 + 2, it1 - 1), 2);
    LSN_WAIT_VM(2 * GROUP);
    __syncthreads();
    read_codes(cq, ca, 0);
    {
      const uint8_t* sa = sA[0] + sa0;
#pragma unroll
      for (int i = 0; i < 8; ++i) af[0][i] = *reinterpret_cast<const bf16x8*>(sa + i * 4096);
#pragma unroll
      for (int j = 0; j < 2; ++j) bq[0][j] = dequant8(cq[j][0], ca[j], pair);
    }
    // Slice t (u = t - it0) sits in stage u % 3.  Each wave's codes and
    // absmax are the rows it loaded itself, so after waiting for its own
    // loads of slice t + 1 (k-step 2; only slice t + 2's may be in flight)
    // it reads slice t + 1's codes without a barrier.  Before k-step 3 all
    // of slice t's activations have been read by this wave (lgkmcnt(0)); the
    // barrier then makes slice t + 1's activations visible and stage u % 3
    // free, and k-step 3 refills it with slice t + 3.
    int st = 0;
    for (int t = it0; t < it1; ++t) {
      const int st1 = st == NST - 1 ? 0 : st + 1;
      kstep(std::integral_constant<int, 0>{}, sA[st] + (sa0 ^ 16), cq, ca, 1, none);
      kstep(std::integral_constant<int, 1>{}, sA[st] + (sa0 ^ 32), cq, ca, 2, none);
      LSN_WAIT_VM(GROUP);
      kstep(std::integral_constant<int, 2>{}, sA[st] + (sa0 ^ 48), cq, ca, 3,
            [&](int s) { if (s == 8) read_codes(cqn, can, st1); });
      __syncthreads();  // (its fence waits lgkmcnt(0): this wave's reads of stage st are done)
      const uint8_t* a_next = gA + min(t + 3, it1 - 1) * (FK * 2);
      const uint8_t* c_next = gC + min(t + 3, it1 - 1) * (FK / 2);
      const uint32_t la = lds_addr(sA[st]) + w * 8 * 1024;
      const uint32_t lc = lds_addr(sC[st]) + w * 2 * 1024;
      const uint32_t lm = lds_addr(&sM[st][w * 64]);
      const uint8_t* m_next = gM + min(t + 3, it1 - 1) * 4;
      kstep(std::integral_constant<int, 3>{}, sA[st1] + sa0, cqn, can, 0, [&](int s) {
        // one M0 per group; the loads address relative to it
        if (s == 0) {
          set_m0(la + 4096);
          dma16_at<-4096>(a_next, offA_o[0]);
        }
        if (s == 1) dma16_at<-3072>(a_next, offA_o[1]);
        if (s == 2) dma16_at<-2048>(a_next, offA_o[2]);
        if (s == 3) dma16_at<-1024>(a_next, offA_o[3]);
        if (s == 4) dma16_at<0>(a_next, offA_o[4]);
        if (s == 5) dma16_at<1024>(a_next, offA_o[5]);
        if (s == 6) dma16_at<2048>(a_next, offA_o[6]);
        if (s == 7) dma16_at<3072>(a_next, offA_o[7]);
        if (s == 8) {
          set_m0(lc);
          dma16_at<0>(c_next, offC_o[0]);
        }
        if (s == 9) dma16_at<1024>(c_next, offC_o[1]);
        if (s == 10) {
          set_m0(lm);
          dma4_at<0>(m_next, offM);
        }
      });
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        cq[j] = cqn[j];
        ca[j] = can[j];
      }
      st = st1;
    }
    LSN_WAIT_VM(0);  // no direct load may still be writing LDS when the waves exit
  }

  // ---- low-rank extension: extra k columns read directly as fragments ----
  const int lk = hh * 8;
  if (p.kext > 0 && blockIdx.y == 0) {
    for (int e0 = 0; e0 < p.kext; e0 += 16) {
      bf16x8 af[8], bfr[2];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = min(m0 + i * 32 + lr, p.M - 1);
        af[i] = *reinterpret_cast<const bf16x8*>(p.Aext + (int64_t)m * p.ldae + e0 + lk);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = min(n0 + w * 64 + j * 32 + lr, p.N - 1);
        bfr[j] = *reinterpret_cast<const bf16x8*>(p.Bext + (int64_t)n * p.ldbe + e0 + lk);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue ----
  // The MFMAs take the weights as their first operand, so tile (i, j) holds
  // y^T: lane (lr, hh) has output row m = m0 + 32i + lr and the columns
  // n = n0 + 64w + 32j + 8g + 4hh + t in acc[i][j][4g + t], i.e. four
  // consecutive columns per 16-byte store.  Fully unrolled for the kernel's
  // output form (MODE -1: raw split-k partial sum).  The output and residual
  // pointers are restrict-qualified: a lane's only same-address pair is one
  // group's own load and store, so this also holds in place (C == R).
  auto epilogue = [&](auto full_) {
    constexpr bool FULL = decltype(full_)::value;
    constexpr bool LOADS = MODE == C_F32_ACC || MODE == C_F32_RES;
    float* const out = MODE < 0 ? p.part + blockIdx.y * p.pstride
                                : reinterpret_cast<float*>(p.C);
    const int64_t ld = MODE < 0 ? (int64_t)p.N : p.ldc;
    const float* const src = MODE == C_F32_RES ? p.R : out;
    const int64_t lds = MODE == C_F32_RES ? p.ldr : ld;
    const int nl = n0 + w * 64 + hh * 4;  // this lane's first column (t = 0, g = 0, j = 0)
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
          const int c = j * 32 + g * 8;  // column offset of this group
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
  if (m0 + FM <= p.M && n0 + FN <= p.N) epilogue(std::true_type{});
  else epilogue(std::false_type{});
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static bool aligned(const void* q, uintptr_t a) { return ((uintptr_t)q & (a - 1)) == 0; }

bool nf4f_eligible(const GemmParams& p, int batch) {
  if (batch != 1 || p.nseg != 1 || p.zdiv != 1 || p.alpha != 1.f || p.causal) return false;
  if (p.M < FM || p.K % FK != 0 || p.rowlen != p.K) return false;
  if (p.lda % 8 != 0 || !aligned(p.A, 16) || !aligned(p.B, 16) || !aligned(p.absmax, 4))
    return false;
  // 16-byte output groups (8-byte for bf16), also for the split-k partials
  if (p.N % 4 != 0 || p.ldc % 4 != 0 || !aligned(p.C, 16) || !aligned(p.part, 16)) return false;
  if (p.cmode == C_F32_RES && (p.ldr % 4 != 0 || !aligned(p.R, 16))) return false;
  if (p.kext > 0 && (p.kext % 16 != 0 || p.ldae % 8 != 0 || p.ldbe % 8 != 0 ||
                     !aligned(p.Aext, 16) || !aligned(p.Bext, 16)))
    return false;
  // 32-bit per-lane offsets
  const int64_t lim = (int64_t)1 << 31;
  return (int64_t)p.M * p.lda < lim && (int64_t)p.N * (p.K / 2) < lim;
}

// One workgroup per CU (512 registers per lane): the k range is split
// so that at most 256 workgroups run, each with at least four slices.
int nf4f_split(int M, int N, int K) {
  const int64_t tiles = (int64_t)((M + FM - 1) / FM) * ((N + FN - 1) / FN);
  if (tiles >= 128) return 1;
  int sp = (int)std::min<int64_t>(8, 256 / tiles);
  sp = std::min(sp, std::max(1, K / FK / 4));
  return std::max(sp, 1);
}

hipError_t nf4f_launch(GemmParams p, hipStream_t s) {
  p.ksplit = nf4f_split(p.M, p.N, p.K);
  p.pstride = split_stride(p.M, p.N);
  if (p.ksplit > 1 && (!p.part || p.part_floats < p.ksplit * p.pstride)) p.ksplit = 1;
  const int tiles = ((p.M + FM - 1) / FM) * ((p.N + FN - 1) / FN);
  const dim3 grid(tiles, p.ksplit, 1);
  if (p.ksplit > 1)
    hipExtLaunchKernelGGL(nf4f_kernel<-1>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32)
    hipExtLaunchKernelGGL(nf4f_kernel<C_F32>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32_ACC)
    hipExtLaunchKernelGGL(nf4f_kernel<C_F32_ACC>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32_RES)
    hipExtLaunchKernelGGL(nf4f_kernel<C_F32_RES>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else
    hipExtLaunchKernelGGL(nf4f_kernel<C_BF16>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  if (p.ksplit > 1) gemm_reduce_launch(p, s);
  return hipGetLastError();
}

}  // namespace lsn
