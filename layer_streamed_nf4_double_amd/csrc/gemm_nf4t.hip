// Input gradient of an NF4 projection, dx = dy W, for full 64-deep K slices,
// built like the forward kernel (gemm_nf4f.hip) around one CDNA4 compute unit.
//
//   C[m, n] (op)= sum_k dy[m, k] * bf16(level[code(k, n)] * absmax(k, n))
//                 (+ the low-rank extension of gemm.hip)
//
// The weight is the same NF4 record the forward pass reads: W^T [K, N], the
// projection's [out, in] matrix, so here K (summed over) is the output
// feature and N the input feature.  Codes sit two per byte along N (even
// element in the low nibble), one fp32 absmax per 64 consecutive elements of
// a row; with N a multiple of 64 each absmax block is 64 columns of one row.
//
// Work split.  A workgroup of four waves owns a 256 x 256 output tile; wave w
// owns all 256 rows and the 64 columns n0 + 64w .. +63, i.e. 8 x 2 tiles of
// v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane), so each weight
// element of the tile is dequantized exactly once per workgroup, directly
// into the B-fragment registers of the wave that uses it.  A fragment holds
// eight consecutive k (weight rows) of one column, while a code byte holds
// two adjacent columns of one row; so lane l of a column-tile pair takes the
// two columns of byte l of the wave's 32-byte row segment: column
// n0 + 64w + 2l in tile 0 and the next one in tile 1.  One byte read and one
// level-pair lookup per weight row then serve both tiles.
//
// K order inside a slice: lane half h takes k = 32h + 8kk .. +7 in k-step kk
// for both operands.
//
// Memory pipeline (one iteration = one slice).  Activations (dy, bf16) move
// exactly as in the forward kernel: direct loads three slices ahead into
// three XOR-swizzled LDS stages, one barrier per slice.  Each wave also
// loads its own weight codes (64 rows x 32 bytes) and the 64 absmax values
// of its column block into LDS only it reads, so they need no barrier.  In a
// wave's code block rows 32..63 start 1056 bytes after rows 0..31: the two
// lane halves read rows k and k + 32 together, and the extra 32 bytes put
// them in different banks.  A k-step reads the code bytes and absmax values
// of the k-step after next, looks up the level pairs of the next one and
// forms its bf16 fragments, all between its MFMAs.
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

constexpr int TM = 256, TN = 256, TK = 64;
constexpr int TST = 3;                   // LDS stages
constexpr int TA_STAGE = TM * TK * 2;    // 32 KiB of activations (bf16)
constexpr int CHALF = 1024 + 32;         // offset of row 32 in a wave's code block
constexpr int CW = CHALF + 1024;         // one wave's code block
constexpr int TGROUP = 8 + 2 + 1;        // direct loads per wave per slice

}  // namespace

// MODE: the output form (C_F32, C_F32_ACC, C_F32_RES, C_BF16), or -1 for the
// raw split-k partial sums.
template <int MODE>
__global__ __launch_bounds__(256) void nf4t_kernel(const GemmParams p) {
  // the level-pair table at LDS address 0 (the largest alignment is placed
  // first): a lookup's address is then just 8 x code byte, one shift of a
  // byte-selected operand (v_lshlrev_b32_sdwa) per byte
  __shared__ __attribute__((aligned(4096))) float2 sPair[256];
  __shared__ __attribute__((aligned(1024))) uint8_t sA[TST][TA_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sC[TST][4 * CW];
  __shared__ __attribute__((aligned(16))) float sM[TST][4][64];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lr = lane & 31, hh = lane >> 5;

  // ---- tile coordinates and k split (XCD-aware, split-major) ----
  const int mt = (p.M + TM - 1) / TM;
  const WorkUnit wu = xcd_unit();
  const int id = wu.tile, ks = wu.split;
  const int m0 = (id % mt) * TM, n0 = (id / mt) * TN;
  const int nw = n0 + 64 * w;                // this wave's first column
  const int nwl = min(nw, p.N - 64);         // the same, kept inside the matrix for loads

  sPair[threadIdx.x] = make_float2(p.levels[threadIdx.x & 15], p.levels[threadIdx.x >> 4]);
  auto pair = [&](uint32_t b8) {  // b8 = 8 * code byte
    return *reinterpret_cast<const float2*>(reinterpret_cast<const char*>(sPair) + b8);
  };

  // ---- direct-load byte offsets of this lane (slice 0) ----
  // activations: as in the forward kernel (load i of wave w fills stage rows
  // (8w + i) * 8 .. +7; lane -> row + lane / 8, physical chunk lane % 8)
  uint32_t offA[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (w * 8 + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    const int row = min(m0 + r, p.M - 1);
    offA[i] = (uint32_t)(((int64_t)row * p.lda + c * 8) * 2);
  }
  // codes: load i fills rows 32i + lane / 2 of the wave's block, half lane % 2
  const int64_t crow = p.N / 2;  // bytes per weight row
  uint32_t offC[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    offC[i] = (uint32_t)((32 * i + (lane >> 1)) * crow + nwl / 2 + 16 * (lane & 1));
  // the same offsets for one M0 per group (instruction offsets 1024 i - 4096
  // for the activations, 0 and CHALF for the codes); never negative, since
  // activation load i covers rows >= 8 i and code load 1 starts at row 32
  // (32 N / 2 >= CHALF for N >= 128)
  uint32_t offA_o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) offA_o[i] = offA[i] + 4096u - 1024u * i;
  const uint32_t offC0 = offC[0], offC1 = offC[1] - (uint32_t)CHALF;
  // absmax: lane -> weight row lane, block nwl / 64
  const int64_t mrow = p.N / 64;  // absmax entries per weight row
  const uint32_t offM = (uint32_t)((lane * mrow + nwl / 64) * 4);

  const uint8_t* gA = reinterpret_cast<const uint8_t*>(p.A);
  const uint8_t* gC = reinterpret_cast<const uint8_t*>(p.B);
  const uint8_t* gM = reinterpret_cast<const uint8_t*>(p.absmax);
  const int64_t cstep = TK * crow;      // code bytes per slice
  const int64_t mstep = TK * mrow * 4;  // absmax bytes per slice

  // split-k: split ks takes slices [it0, it1)
  const int nkt = p.K / TK;
  const int kper = (nkt + p.ksplit - 1) / p.ksplit;
  const int it0 = min(nkt, ks * kper), it1 = min(nkt, it0 + kper);

  // the TGROUP direct loads of slice it into LDS stage st
  auto issue = [&](int it, int st) {
    const uint8_t* a = gA + it * (TK * 2);
    const uint32_t la = lds_addr(sA[st]) + w * 8 * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(a, offA[i], la + i * 1024);
    const uint8_t* c = gC + it * cstep;
    const uint32_t lc = lds_addr(sC[st]) + w * CW;
    dma16(c, offC[0], lc);
    dma16(c, offC[1], lc + CHALF);
    dma4(gM + it * mstep, offM, lds_addr(&sM[st][w][0]));
  };

  // ---- per-lane LDS read offsets ----
  // activation fragment of row tile i, k-step kk: row i*32 + lr, logical chunk
  // 4*hh + kk -> physical (4*hh ^ swz(lr)) ^ kk
  const int sa0 = lr * 128 + (((4 * hh) ^ swz(lr)) * 16);
  // code byte lr of weight row 32*hh (+ 8*kk + e) of the wave's block
  const int sc0 = w * CW + hh * CHALF + lr;

  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  bf16x8 af[2][8];    // activation fragments, double buffered over k-steps
  bf16x8 bq[2][2];    // weight fragments [kk & 1][column tile]
  uint32_t cb[2][8];  // code bytes of a k-step's eight rows [set][row]
  f32x4 am[2][2];     // absmax of those rows [set][row / 4]

  // code bytes and absmax of k-step kk (of its slice) from stage st into set S
  auto read_bytes = [&](auto S_, int st, auto kk_, int e) {
    constexpr int S = decltype(S_)::value, kk = decltype(kk_)::value;
    cb[S][e] = sC[st][sc0 + (8 * kk + e) * 32];
    if (e == 0 || e == 4)
      am[S][e >> 2] = *reinterpret_cast<const f32x4*>(&sM[st][w][32 * hh + 8 * kk + e]);
  };
  // fragments of both column tiles from looked-up level pairs lo/hi and set S
  auto pack_pair = [&](auto S_, const float (&lv)[8], int pp) {
    constexpr int S = decltype(S_)::value;
    const float a0 = am[S][pp >> 1][(2 * pp) & 3], a1 = am[S][pp >> 1][(2 * pp + 1) & 3];
    return pack_bf16x2(lv[2 * pp] * a0, lv[2 * pp + 1] * a1);
  };

  // One k-step as 16 MFMA slots (row tile s/2, column tile s%2).  Between
  // them, in a fixed order (sched_barrier after every slot): the next
  // k-step's activation fragments and level-pair lookups (slots 0-7), its
  // products and bf16 packing, and the code bytes and absmax of the k-step
  // after next (slots 8-15), from stage stn.  extra(s) adds per-slot work.
  auto kstep = [&](auto kk_, const uint8_t* an, int stn, auto extra) {
    constexpr int kk = decltype(kk_)::value;
    constexpr int F = kk & 1;           // this k-step's fragments
    constexpr int NX = F ^ 1;           // byte set of the next k-step
    constexpr int K2 = (kk + 2) & 3;    // the k-step after next, within its slice
    float lo[8], hi[8];
    u32x4 r0, r1;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      acc[s >> 1][s & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          bq[F][s & 1], af[F][s >> 1], acc[s >> 1][s & 1], 0, 0, 0);
      if (s < 8) {
        af[F ^ 1][s] = *reinterpret_cast<const bf16x8*>(an + s * 4096);
        const float2 l = pair(cb[NX][s] << 3);
        lo[s] = l.x;
        hi[s] = l.y;
      } else {
        const int pp = (s - 8) & 3;
        if (s < 12) r0[pp] = pack_pair(std::integral_constant<int, NX>{}, lo, pp);
        else r1[pp] = pack_pair(std::integral_constant<int, NX>{}, hi, pp);
        if (s == 11) bq[F ^ 1][0] = __builtin_bit_cast(bf16x8, r0);
        if (s == 15) bq[F ^ 1][1] = __builtin_bit_cast(bf16x8, r1);
        read_bytes(std::integral_constant<int, F>{}, stn, std::integral_constant<int, K2>{}, s - 8);
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
    LSN_WAIT_VM(2 * TGROUP);
    __syncthreads();
    // k-step 0's fragments; the code bytes of k-step 1 wait in set 1
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      read_bytes(std::integral_constant<int, 0>{}, 0, std::integral_constant<int, 0>{}, e);
      read_bytes(std::integral_constant<int, 1>{}, 0, std::integral_constant<int, 1>{}, e);
    }
    {
      const uint8_t* sa = sA[0] + sa0;
#pragma unroll
      for (int i = 0; i < 8; ++i) af[0][i] = *reinterpret_cast<const bf16x8*>(sa + i * 4096);
      float lo[8], hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 l = pair(cb[0][e] << 3);
        lo[e] = l.x;
        hi[e] = l.y;
      }
      u32x4 r0, r1;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        r0[pp] = pack_pair(std::integral_constant<int, 0>{}, lo, pp);
        r1[pp] = pack_pair(std::integral_constant<int, 0>{}, hi, pp);
      }
      bq[0][0] = __builtin_bit_cast(bf16x8, r0);
      bq[0][1] = __builtin_bit_cast(bf16x8, r1);
    }
    // Slice t (u = t - it0) sits in stage u % 3.  K-steps 0 and 1 read the
    // code bytes of k-steps 2 and 3 (stage of t); k-steps 2 and 3 those of
    // slice t + 1's k-steps 0 and 1, after this wave has waited for its own
    // loads of slice t + 1 (only slice t + 2's may still be in flight).
    // The barrier before k-step 3 makes slice t + 1's activations visible
    // and frees stage u % 3 (every wave has read its activations, and this
    // wave its codes), and k-step 3 refills it with slice t + 3.
    int st = 0;
    for (int t = it0; t < it1; ++t) {
      const int st1 = st == TST - 1 ? 0 : st + 1;
      kstep(std::integral_constant<int, 0>{}, sA[st] + (sa0 ^ 16), st, none);
      kstep(std::integral_constant<int, 1>{}, sA[st] + (sa0 ^ 32), st, none);
      LSN_WAIT_VM(TGROUP);
      kstep(std::integral_constant<int, 2>{}, sA[st] + (sa0 ^ 48), st1, none);
      __syncthreads();  // (its fence waits lgkmcnt(0): this wave's reads of stage st are done)
      const int tn = min(t + 3, it1 - 1);
      const uint8_t* a_next = gA + tn * (TK * 2);
      const uint8_t* c_next = gC + tn * cstep;
      const uint8_t* m_next = gM + tn * mstep;
      const uint32_t la = lds_addr(sA[st]) + w * 8 * 1024;
      const uint32_t lc = lds_addr(sC[st]) + w * CW;
      const uint32_t lm = lds_addr(&sM[st][w][0]);
      kstep(std::integral_constant<int, 3>{}, sA[st1] + sa0, st1, [&](int s) {
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
          dma16_at<0>(c_next, offC0);
        }
        if (s == 9) dma16_at<CHALF>(c_next, offC1);
        if (s == 10) {
          set_m0(lm);
          dma4_at<0>(m_next, offM);
        }
      });
      st = st1;
    }
    LSN_WAIT_VM(0);  // no direct load may still be writing LDS when the waves exit
  }

  // ---- low-rank extension: extra k columns read directly as fragments ----
  const int lk = hh * 8;
  if (p.kext > 0 && ks == 0) {
    for (int e0 = 0; e0 < p.kext; e0 += 16) {
      bf16x8 ax[8], bx[2];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = min(m0 + i * 32 + lr, p.M - 1);
        ax[i] = *reinterpret_cast<const bf16x8*>(p.Aext + (int64_t)m * p.ldae + e0 + lk);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = min(nw + 2 * lr + j, p.N - 1);
        bx[j] = *reinterpret_cast<const bf16x8*>(p.Bext + (int64_t)n * p.ldbe + e0 + lk);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bx[j], ax[i], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue ----
  // Tile (i, j) holds the transpose: lane (lr, hh) has output row
  // m = m0 + 32i + lr, and B-lane 8g + 4hh + t, i.e. column
  // nw + 16g + 8hh + 2t + j, in acc[i][j][4g + t].  Interleaving the two
  // column tiles gives eight consecutive columns per (i, g): two 16-byte
  // stores (one for bf16).  N is a multiple of 64, so a wave's columns are
  // all inside the matrix or all outside.
  auto epilogue = [&](auto full_) {
    constexpr bool FULL = decltype(full_)::value;
    constexpr bool LOADS = MODE == C_F32_ACC || MODE == C_F32_RES;
    if (!FULL && nw >= p.N) return;
    float* const out = MODE < 0 ? p.part + ks * p.pstride
                                : reinterpret_cast<float*>(p.C);
    const int64_t ld = MODE < 0 ? (int64_t)p.N : p.ldc;
    const float* const src = MODE == C_F32_RES ? p.R : out;
    const int64_t lds = MODE == C_F32_RES ? p.ldr : ld;
    const int nl = nw + hh * 8;  // this lane's first column (g = 0)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = m0 + i * 32 + lr;
      if (!FULL && m >= p.M) continue;
      float* __restrict__ orow = out + (int64_t)m * ld + nl;
      uint16_t* __restrict__ brow = reinterpret_cast<uint16_t*>(p.C) + (int64_t)m * ld + nl;
      const float* __restrict__ srow = src + (int64_t)m * lds + nl;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = g * 16;  // column offset of this group
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
  if (m0 + TM <= p.M && n0 + TN <= p.N) epilogue(std::true_type{});
  else epilogue(std::false_type{});
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static bool aligned16(const void* q) { return ((uintptr_t)q & 15) == 0; }

bool nf4t_eligible(const GemmParams& p, int batch) {
  if (batch != 1 || p.nseg != 1 || p.zdiv != 1 || p.alpha != 1.f || p.causal) return false;
  if (p.M < TM || p.K % TK != 0 || p.rowlen != p.N || p.N % 64 != 0 || p.N < 128) return false;
  if (p.lda % 8 != 0 || !aligned16(p.A) || !aligned16(p.B) || ((uintptr_t)p.absmax & 3) != 0)
    return false;
  // 16-byte output groups of eight columns (bf16) or four (fp32), also for the partials
  if (p.ldc % 8 != 0 || !aligned16(p.C) || !aligned16(p.part)) return false;
  if (p.cmode == C_F32_RES && (p.ldr % 4 != 0 || !aligned16(p.R))) return false;
  if (p.kext > 0 && (p.kext % 16 != 0 || p.ldae % 8 != 0 || p.ldbe % 8 != 0 ||
                     !aligned16(p.Aext) || !aligned16(p.Bext)))
    return false;
  // 32-bit per-lane offsets (the weight offsets stay inside one 64-row slice)
  return (int64_t)p.M * p.lda < ((int64_t)1 << 31);
}

hipError_t nf4t_launch(GemmParams p, hipStream_t s) {
  p.ksplit = nf4f_split(p.M, p.N, p.K);
  p.pstride = split_stride(p.M, p.N);
  if (p.ksplit > 1 && (!p.part || p.part_floats < p.ksplit * p.pstride)) p.ksplit = 1;
  const int tiles = ((p.M + TM - 1) / TM) * ((p.N + TN - 1) / TN);
  const dim3 grid(tiles, p.ksplit, 1);
  if (p.ksplit > 1)
    hipExtLaunchKernelGGL(nf4t_kernel<-1>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32)
    hipExtLaunchKernelGGL(nf4t_kernel<C_F32>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32_ACC)
    hipExtLaunchKernelGGL(nf4t_kernel<C_F32_ACC>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32_RES)
    hipExtLaunchKernelGGL(nf4t_kernel<C_F32_RES>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  else
    hipExtLaunchKernelGGL(nf4t_kernel<C_BF16>, grid, dim3(256), 0, s, p.ev0, p.ev1, 0, p);
  if (p.split_used) *p.split_used = p.ksplit;
  if (p.ksplit > 1 && !p.defer_reduce) gemm_reduce_launch(p, s);
  return hipGetLastError();
}

}  // namespace lsn
