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
// Work split.  A workgroup of four waves (one per SIMD) owns a 256 x 128 NT
// output tile (NT = 2: 256 x 256; NT = 1: 256 x 128, for narrow projections);
// wave w owns all 256 rows and the 32 NT columns n0 + 32 NT w .. , i.e. 8 x NT
// tiles of v_mfma_f32_32x32x16_bf16 (128 NT fp32 accumulators per lane).
// Because the waves split only the N dimension, each weight element of the
// tile is dequantized exactly once per workgroup, directly into the
// B-fragment registers of the wave that uses it; the dequantized weight never
// passes through LDS.  Only the activation slice [256 x 64] is shared through
// LDS: 0.5 (NT = 2) or 1 (NT = 1) KiB of LDS reads per MFMA.
//
// Tile choice (nf4f_plan).  A narrow projection at a few hundred tokens has
// few 256 x 256 tiles (32 at 512 x 4096 -> 4096), so filling 256 compute
// units takes an 8-way k split whose fp32 partial sums (8 copies of the
// output) cost more than the MFMAs.  The 256 x 128 tile doubles the tile
// count and halves the split and its partial-sum traffic, at twice the LDS
// reads per MFMA (about half the measured LDS bandwidth).
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
// Producer wave (256 x 128 tile).  With one wave per SIMD every instruction
// a wave issues sits in line with its MFMAs, and a slice's eleven direct
// loads per wave cost its last k-step about 200 cycles (clock stamps).  The
// 256 x 128 form therefore runs a fifth wave that issues every direct load
// of the workgroup (32 activation, 4 code, 4 absmax per slice), waits for
// them and meets the four MFMA waves at the same one barrier per slice; the
// MFMA waves issue no memory instruction in the main loop and read the next
// slice's codes after that barrier, at the start of the last k-step.  (Its
// 208 registers let a second wave share one SIMD; the 256 x 256 form, with
// 256 accumulators per lane, keeps one wave per SIMD and its own loads.)
//
// SwiGLU epilogue (C_SWIGLU, 256 x 256 tile only).  The weight is the fused
// gate|up record [2F, K]; a tile then covers gate columns n0 .. n0+127 and
// the same up columns F+n0 .. F+n0+127: wave w's column tile 0 holds gate
// columns n0+32w .., tile 1 the up columns of the same features, so each
// lane has gate and up of the same (m, f) in matching accumulators and
// writes a = bf16(silu(gate) * up) [M, F] directly (a quarter of the bytes of
// the fp32 gate|up output, and no separate SwiGLU pass).
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

constexpr int FM = 256, FK = 64;
constexpr int NST = 3;                 // LDS stages
constexpr int A_STAGE = FM * FK * 2;   // 32 KiB of activations (bf16)
// per column-tile count NT: tile width, codes per stage, direct loads per
// wave per slice (8 activation, NT code, 1 absmax)
template <int NT> struct Shape {
  static constexpr int FN = 128 * NT;
  static constexpr int C_STAGE = FN * FK / 2;
  static constexpr int GROUP = 8 + NT + 1;
};

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
template <int MODE, int NT>
__global__ __launch_bounds__(NT == 1 ? 320 : 256) void nf4f_kernel(const GemmParams p) {
  // NT = 1: a fifth wave issues every direct load of the workgroup (the
  // producer); the four MFMA waves issue none in the main loop
  constexpr bool PW = NT == 1;
  constexpr int GP = 32 + 4 + 4;  // producer loads per slice
  constexpr int FN = Shape<NT>::FN, C_STAGE = Shape<NT>::C_STAGE, GROUP = Shape<NT>::GROUP;
  constexpr int NS = 8 * NT;  // MFMA slots per k-step
  constexpr bool SW = MODE == C_SWIGLU;
  static_assert(!SW || NT == 2, "the SwiGLU epilogue pairs two column tiles per wave");
  constexpr int TN = SW ? FN / 2 : FN;  // output columns per tile
  // the level-pair table at LDS address 0 (the largest alignment is placed
  // first): a lookup's address is then just 8 x code byte, one shift of a
  // byte-selected operand (v_lshlrev_b32_sdwa) per byte
  __shared__ __attribute__((aligned(4096))) float2 sPair[256];
  __shared__ __attribute__((aligned(1024))) uint8_t sA[NST][A_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sC[NST][C_STAGE];
  // absmax: 64 entries per wave (rows beyond its 32 NT columns are unused)
  __shared__ __attribute__((aligned(1024))) float sM[NST][4 * 64];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lr = lane & 31, hh = lane >> 5;

  // ---- tile coordinates and k split (XCD-aware, split-major) ----
  const int mt = (p.M + FM - 1) / FM;
  const WorkUnit wu = xcd_unit();
  const int id = wu.tile, ks = wu.split;
  const int m0 = (id % mt) * FM, n0 = (id / mt) * TN;
  const int Fh = p.N / 2;  // SwiGLU: the feature count F
  // weight row (W^T row, clamped into the matrix) of row rr of wave w's
  // column tile j
  auto wrow = [&](int j, int rr) {
    if constexpr (SW) return j * Fh + min(n0 + 32 * w + rr, Fh - 1);
    else return min(n0 + 32 * NT * w + 32 * j + rr, p.N - 1);
  };

  // entry b: the levels of code byte b (low nibble: even element, high
  // nibble: odd element); one 8-byte read dequantizes two elements
  if (threadIdx.x < 256)
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
  // codes: load i of wave w fills weight rows (NT w + i) * 32 .. +31 (32 B
  // each); lane -> row + lane / 2, physical half lane % 2
  uint32_t offC[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int r = (w * NT + i) * 32 + (lane >> 1);
    const int h = (lane & 1) ^ ((r >> 3) & 1);
    offC[i] = (uint32_t)((int64_t)wrow(i, lane >> 1) * (p.K / 2) + h * 16);
  }
  // the same offsets for loads at instruction offset 1024 i - 4096 from one
  // M0 (activation load i) and at 1024 i (code load i); never negative,
  // since load i covers rows >= 8 i (activations) or >= 32 i (codes)
  uint32_t offA_o[8], offC_o[NT];
#pragma unroll
  for (int i = 0; i < 8; ++i) offA_o[i] = offA[i] + 4096u - 1024u * i;
#pragma unroll
  for (int i = 0; i < NT; ++i) offC_o[i] = offC[i] - 1024u * i;
  // absmax: wave w fills its 64-entry region with the rows of its column
  // tiles (entry 32 j + rr: row rr of tile j; with NT = 1 the upper half is
  // unused)
  const uint32_t offM = (uint32_t)((int64_t)wrow(lane >> 5, lane & 31) * (p.K / FK) * 4);

  const uint8_t* gA = reinterpret_cast<const uint8_t*>(p.A);
  const uint8_t* gC = reinterpret_cast<const uint8_t*>(p.B);
  const uint8_t* gM = reinterpret_cast<const uint8_t*>(p.absmax);

  // split-k: split ks takes slices [it0, it1)
  const int nkt = p.K / FK;
  const int kper = (nkt + p.ksplit - 1) / p.ksplit;
  const int it0 = min(nkt, ks * kper), it1 = min(nkt, it0 + kper);

  // the GROUP direct loads of slice it into LDS stage st
  auto issue = [&](int it, int st) {
    const uint8_t* a = gA + it * (FK * 2);
    const uint32_t la = lds_addr(sA[st]) + w * 8 * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(a, offA[i], la + i * 1024);
    const uint8_t* c = gC + it * (FK / 2);
    const uint32_t lc = lds_addr(sC[st]) + w * NT * 1024;
#pragma unroll
    for (int i = 0; i < NT; ++i) dma16(c, offC[i], lc + i * 1024);
    dma4(gM + it * 4, offM, lds_addr(&sM[st][w * 64]));
  };

  if constexpr (PW) {
    if (w == 4) {  // ---- the producer ----
      // activation load i fills stage rows 8 i .. 8 i + 7 (lane -> row + lane
      // / 8, physical chunk lane % 8); eight loads per M0 at offsets 1024 i -
      // 4096, so the per-lane offsets have that subtracted
      uint32_t oA[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int r = i * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        const int row = min(m0 + r, p.M - 1);
        oA[i] = (uint32_t)(((int64_t)row * p.lda + c * 8) * 2) + 4096u - 1024u * (i & 7);
      }
      // code load i fills MFMA wave i's 32 rows (lane -> row + lane / 2,
      // physical half lane % 2); absmax load i fills wave i's 64-entry region
      uint32_t oC[4], oM[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i * 32 + (lane >> 1);
        const int h = (lane & 1) ^ ((r >> 3) & 1);
        oC[i] = (uint32_t)((int64_t)min(n0 + 32 * i + (lane >> 1), p.N - 1) * (p.K / 2) + h * 16);
        oM[i] = (uint32_t)((int64_t)min(n0 + 32 * i + lane, p.N - 1) * (p.K / FK) * 4);
      }
      const uint8_t* gA = reinterpret_cast<const uint8_t*>(p.A);
      const uint8_t* gC = reinterpret_cast<const uint8_t*>(p.B);
      const uint8_t* gM = reinterpret_cast<const uint8_t*>(p.absmax);
      const int nkt = p.K / FK;
      const int kper = (nkt + p.ksplit - 1) / p.ksplit;
      const int it0 = min(nkt, ks * kper), it1 = min(nkt, it0 + kper);
      if (it1 <= it0) return;  // (the MFMA waves then take no barrier either)
      auto pissue = [&](int it, int st) {
        const uint8_t* a = gA + it * (FK * 2);
        const uint32_t la = lds_addr(sA[st]);
        auto a8 = [&](auto g_) {
          constexpr int g = decltype(g_)::value;
          set_m0(la + g * 8192 + 4096);
          dma16_at<-4096>(a, oA[8 * g + 0]);
          dma16_at<-3072>(a, oA[8 * g + 1]);
          dma16_at<-2048>(a, oA[8 * g + 2]);
          dma16_at<-1024>(a, oA[8 * g + 3]);
          dma16_at<0>(a, oA[8 * g + 4]);
          dma16_at<1024>(a, oA[8 * g + 5]);
          dma16_at<2048>(a, oA[8 * g + 6]);
          dma16_at<3072>(a, oA[8 * g + 7]);
        };
        a8(std::integral_constant<int, 0>{});
        a8(std::integral_constant<int, 1>{});
        a8(std::integral_constant<int, 2>{});
        a8(std::integral_constant<int, 3>{});
        const uint8_t* c = gC + it * (FK / 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(c, oC[i], lds_addr(sC[st]) + i * 1024);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma4(gM + it * 4, oM[i], lds_addr(&sM[st][i * 64]));
      };
      // slices it0, it0 + 1 (clamped); slice it0 landed; then it0 + 2
      pissue(it0, 0);
      pissue(min(it0 + 1, it1 - 1), 1);
      LSN_WAIT_VM(GP);
      pissue(min(it0 + 2, it1 - 1), 2);
      __syncthreads();
      int st = 0;
      for (int t = it0; t < it1; ++t) {
        LSN_WAIT_VM(GP);  // slice t + 1 landed (only slice t + 2's loads in flight)
        __syncthreads();  // the MFMA waves are done with stage st
        pissue(min(t + 3, it1 - 1), st);
        st = st == NST - 1 ? 0 : st + 1;
      }
      LSN_WAIT_VM(0);
      return;
    }
  }

  // ---- per-lane LDS read offsets ----
  // activation fragment of row tile i, k-step kk: row i*32 + lr, logical chunk
  // 4*hh + kk -> physical (4*hh ^ swz(lr)) ^ kk (kk only flips the low bits)
  const int sa0 = lr * 128 + (((4 * hh) ^ swz(lr)) * 16);
  // codes of column tile j: row 32 NT w + 32j + lr, logical half hh
  const int sc0 = (w * 32 * NT + lr) * 32 + ((hh ^ ((lr >> 3) & 1)) * 16);
  const int sm0 = w * 64 + lr;

  f32x16 acc[8][NT];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  bf16x8 af[2][8];   // activation fragments, double buffered over k-steps
  bf16x8 bq[2][NT];  // weight fragments [kk & 1][j]
  u32x4 cq[NT], cqn[NT];  // codes of this slice and of the next one (per column tile)
  float ca[NT], can[NT];

  auto read_codes = [&](u32x4 (&q)[NT], float (&a)[NT], int st) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      q[j] = *reinterpret_cast<const u32x4*>(sC[st] + sc0 + j * 1024);
      a[j] = sM[st][sm0 + j * 32];
    }
  };

  // One k-step as 8 NT MFMA slots (row tile s / NT, column tile s % NT).
  // Between them, in a fixed order (sched_barrier after every slot): the next
  // k-step's eight activation fragments (slots 0-7) and the 4 NT level-pair
  // reads of its weight tiles (slots 0 .. 4 NT - 1), then the products and
  // bf16 packing (slots 4 NT .. 8 NT - 1, when the reads have long returned).
  // extra(s) adds per-slot work (the direct loads of the last k-step).
  auto kstep = [&](auto kk_, const uint8_t* an, const u32x4 (&q)[NT], const float (&a)[NT],
                   int kn, auto extra) {
    constexpr int F = decltype(kk_)::value & 1;
    float lvv[NT][8];
    u32x4 r[NT];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      acc[s / NT][s % NT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          bq[F][s % NT], af[F][s / NT], acc[s / NT][s % NT], 0, 0, 0);
      if (s < 8) af[F ^ 1][s] = *reinterpret_cast<const bf16x8*>(an + s * 4096);
      if (s < 4 * NT) {  // level pair ph of tile jt (byte ph of the code word)
        const int jt = s >> 2, ph = s & 3;
        const float2 l = pair(pair_off(q[jt][kn], ph));
        lvv[jt][2 * ph] = l.x;
        lvv[jt][2 * ph + 1] = l.y;
      } else {
        const int jt = (s - 4 * NT) >> 2, pp = (s - 4 * NT) & 3;
        r[jt][pp] = pack_bf16x2(lvv[jt][2 * pp] * a[jt], lvv[jt][2 * pp + 1] * a[jt]);
        if (pp == 3) bq[F ^ 1][jt] = __builtin_bit_cast(bf16x8, r[jt]);
      }
      extra(s);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto none = [](int) {};
  // PW, the last k-step of a slice (k-step 3, after the barrier): the next
  // slice's codes are read here (slot 0), their level pairs in slots 2-3 and
  // the products in slots 5-6, so the next k-step's weight fragment is ready
  auto kstep3pw = [&](const uint8_t* an, int st1) {
    float lvv[8];
    u32x4 r;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      acc[s][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bq[1][0], af[1][s], acc[s][0], 0, 0, 0);
      af[0][s] = *reinterpret_cast<const bf16x8*>(an + s * 4096);
      if (s == 0) read_codes(cqn, can, st1);
      if (s == 2 || s == 3) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int ph = 2 * (s - 2) + u;
          const float2 l = pair(pair_off(cqn[0][0], ph));
          lvv[2 * ph] = l.x;
          lvv[2 * ph + 1] = l.y;
        }
      }
      if (s == 5 || s == 6) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int pp = 2 * (s - 5) + u;
          r[pp] = pack_bf16x2(lvv[2 * pp] * can[0], lvv[2 * pp + 1] * can[0]);
        }
        if (s == 6) bq[0][0] = __builtin_bit_cast(bf16x8, r);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- low-rank extension: extra k columns read directly as fragments ----
  // (split 0 only), added before the main loop: its loads are issued after
  // the prologue's direct loads and land with them
  auto extension = [&]() {
    const int lk = hh * 8;
    for (int e0 = 0; e0 < p.kext; e0 += 16) {
      bf16x8 xf[8], bfr[NT];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = min(m0 + i * 32 + lr, p.M - 1);
        xf[i] = *reinterpret_cast<const bf16x8*>(p.Aext + (int64_t)m * p.ldae + e0 + lk);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(p.Bext + (int64_t)wrow(j, lr) * p.ldbe + e0 + lk);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], xf[i], acc[i][j], 0, 0, 0);
    }
  };
  const bool ext = p.kext > 0 && ks == 0;

  if (it1 > it0) {
    // prologue: slices it0 .. it0+2 (clamped) into stages 0 .. 2
    if constexpr (!PW) {
      issue(it0, 0);
      issue(min(it0 + 1, it1 - 1), 1);
      issue(min(it0 + 2, it1 - 1), 2);
    }
    if (ext) extension();
    if constexpr (!PW) LSN_WAIT_VM(2 * GROUP);
    __syncthreads();
    read_codes(cq, ca, 0);
    {
      const uint8_t* sa = sA[0] + sa0;
#pragma unroll
      for (int i = 0; i < 8; ++i) af[0][i] = *reinterpret_cast<const bf16x8*>(sa + i * 4096);
#pragma unroll
      for (int j = 0; j < NT; ++j) bq[0][j] = dequant8(cq[j][0], ca[j], pair);
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
      if constexpr (PW) {
        kstep(std::integral_constant<int, 2>{}, sA[st] + (sa0 ^ 48), cq, ca, 3, none);
        __syncthreads();  // slice t + 1 landed (the producer waited); stage st is free
        kstep3pw(sA[st1] + sa0, st1);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          cq[j] = cqn[j];
          ca[j] = can[j];
        }
        st = st1;
        continue;
      }
      LSN_WAIT_VM(GROUP);
      kstep(std::integral_constant<int, 2>{}, sA[st] + (sa0 ^ 48), cq, ca, 3,
            [&](int s) { if (s == 4 * NT) read_codes(cqn, can, st1); });
      __syncthreads();  // (its fence waits lgkmcnt(0): this wave's reads of stage st are done)
      const uint8_t* a_next = gA + min(t + 3, it1 - 1) * (FK * 2);
      const uint8_t* c_next = gC + min(t + 3, it1 - 1) * (FK / 2);
      const uint32_t la = lds_addr(sA[st]) + w * 8 * 1024;
      const uint32_t lc = lds_addr(sC[st]) + w * NT * 1024;
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
        // codes and absmax: in slots 8-10 of a 16-slot k-step, after the
        // last activation load in an 8-slot one
        if (s == (NT == 2 ? 8 : 7)) {
          set_m0(lc);
          dma16_at<0>(c_next, offC_o[0]);
        }
        if constexpr (NT == 2)
          if (s == 9) dma16_at<1024>(c_next, offC_o[NT - 1]);
        if (s == (NT == 2 ? 10 : 7)) {
          set_m0(lm);
          dma4_at<0>(m_next, offM);
        }
      });
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        cq[j] = cqn[j];
        ca[j] = can[j];
      }
      st = st1;
    }
    LSN_WAIT_VM(0);  // no direct load may still be writing LDS when the waves exit
  } else if (ext) {
    extension();
  }

  // ---- epilogue ----
  // The MFMAs take the weights as their first operand, so tile (i, j) holds
  // y^T: lane (lr, hh) has output row m = m0 + 32i + lr and the columns
  // n = n0 + 64w + 32j + 8g + 4hh + t in acc[i][j][4g + t], i.e. four
  // consecutive columns per 16-byte store (n = n0 + 32 NT w + ... in
  // general).  Fully unrolled for the kernel's
  // output form (MODE -1: raw split-k partial sum).  The output and residual
  // pointers are restrict-qualified: a lane's only same-address pair is one
  // group's own load and store, so this also holds in place (C == R).
  auto epilogue = [&](auto full_) {
    constexpr bool FULL = decltype(full_)::value;
    if constexpr (SW) {  // a[m][f] for f = n0 + 32w + 8g + 4hh + t
      const int fl = n0 + 32 * w + hh * 4;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = m0 + i * 32 + lr;
        if (!FULL && m >= p.M) continue;
        uint16_t* __restrict__ arow = reinterpret_cast<uint16_t*>(p.C) + (int64_t)m * p.ldc + fl;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (!FULL && fl + g * 8 >= Fh) continue;
          float r[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) r[t] = swiglu_act(acc[i][0][4 * g + t], acc[i][1][4 * g + t]);
          *reinterpret_cast<u32x2*>(arow + g * 8) = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
        }
      }
    } else {
      constexpr bool LOADS = MODE == C_F32_ACC || MODE == C_F32_RES;
      float* const out = MODE < 0 ? p.part + ks * p.pstride
                                  : reinterpret_cast<float*>(p.C);
      const int64_t ld = MODE < 0 ? (int64_t)p.N : p.ldc;
      const float* const src = MODE == C_F32_RES ? p.R : out;
      const int64_t lds = MODE == C_F32_RES ? p.ldr : ld;
      const int nl = n0 + w * 32 * NT + hh * 4;  // this lane's first column (t = 0, g = 0, j = 0)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = m0 + i * 32 + lr;
        if (!FULL && m >= p.M) continue;
        float* __restrict__ orow = out + (int64_t)m * ld + nl;
        uint16_t* __restrict__ brow = reinterpret_cast<uint16_t*>(p.C) + (int64_t)m * ld + nl;
        const float* __restrict__ srow = src + (int64_t)m * lds + nl;
#pragma unroll
        for (int j = 0; j < NT; ++j)
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
    }
  };
  if (m0 + FM <= p.M && (SW ? n0 + TN <= Fh : n0 + FN <= p.N)) epilogue(std::true_type{});
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
// so that at most 256 workgroups run, each with at least four slices.  This
// is the split of the 256 x 256 tile (both NF4 kernels use it).
static int split_for(int64_t tiles, int K);
int nf4f_split(int M, int N, int K) {
  return split_for((int64_t)((M + FM - 1) / FM) * ((N + 255) / 256), K);
}

// The forward kernel's tile and split: the tile width (256 or 128 columns)
// and split (1..8, at least four slices per workgroup) with the lowest
// modelled time
//   rounds of 256 workgroups x slices per workgroup x time per slice
//   + split-k partial sums: written once, read and added once, the sum
//     written once ((2 split + 1) M N 4 bytes),
// with times measured on MI355X at one workgroup per CU: 1.70 us per slice
// of a 256 x 256 tile, 1.09 us of a 256 x 128 tile, 0.25 us per MB of
// partial-sum traffic.  (512 tokens: 4096 -> 4096 ran 45 us on the wide tile
// split 8, 36 us on the narrow one split 4; 4096 -> 14336 81 us split 2
// against 71 us unsplit; 1024 tokens, 14336 -> 4096: 129 us wide, 135 us
// narrow.)
static int split_for(int64_t tiles, int K) {
  if (tiles >= 128) return 1;
  int sp = (int)std::min<int64_t>(8, std::max<int64_t>(1, 256 / tiles));
  sp = std::min(sp, std::max(1, K / FK / 4));
  return std::max(sp, 1);
}

static double plan_cost(int M, int N, int K, int nt, int split) {
  const int64_t tiles = (int64_t)((M + FM - 1) / FM) * ((N + 128 * nt - 1) / (128 * nt));
  const double rounds = (double)((tiles * split + 255) / 256);
  const double slices = (double)((K / FK + split - 1) / split);
  double us = rounds * slices * (nt == 2 ? 1.70 : 1.09);
  if (split > 1) us += (2.0 * split + 1.0) * (double)M * N * 4.0 * 0.25e-6;
  return us;
}

bool nf4f_swiglu_ok(const GemmParams& p) {
  if (p.cmode != C_SWIGLU || p.N % 8 != 0 || p.ldc % 4 != 0 || !nf4f_eligible(p, 1)) return false;
  const Nf4fPlan plan = nf4f_plan(p.M, p.N, p.K);
  return plan.nt == 2 && plan.split == 1;
}

Nf4fPlan nf4f_plan(int M, int N, int K) {
  Nf4fPlan best{2, 1};
  double cost = plan_cost(M, N, K, 2, 1);
  for (int nt = 2; nt >= 1; --nt)
    for (int sp = 1; sp <= 8 && (sp == 1 || K / FK / sp >= 4); ++sp) {
      const double c = plan_cost(M, N, K, nt, sp);
      if (c < cost) {
        cost = c;
        best = {nt, sp};
      }
    }
  return best;
}

template <int NT>
static void nf4f_launch_t(const GemmParams& p, hipStream_t s) {
  const int tiles = ((p.M + FM - 1) / FM) * ((p.N + Shape<NT>::FN - 1) / Shape<NT>::FN);
  const dim3 grid(tiles, p.ksplit, 1);
  const dim3 blk(NT == 1 ? 320 : 256);
  if (p.ksplit > 1)
    hipExtLaunchKernelGGL((nf4f_kernel<-1, NT>), grid, blk, 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32)
    hipExtLaunchKernelGGL((nf4f_kernel<C_F32, NT>), grid, blk, 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32_ACC)
    hipExtLaunchKernelGGL((nf4f_kernel<C_F32_ACC, NT>), grid, blk, 0, s, p.ev0, p.ev1, 0, p);
  else if (p.cmode == C_F32_RES)
    hipExtLaunchKernelGGL((nf4f_kernel<C_F32_RES, NT>), grid, blk, 0, s, p.ev0, p.ev1, 0, p);
  else
    hipExtLaunchKernelGGL((nf4f_kernel<C_BF16, NT>), grid, blk, 0, s, p.ev0, p.ev1, 0, p);
}

hipError_t nf4f_launch(GemmParams p, hipStream_t s) {
  if (p.cmode == C_SWIGLU) {  // one unsplit launch, tiles of 128 features
    if (!nf4f_swiglu_ok(p)) return hipErrorInvalidValue;
    const int tiles = ((p.M + FM - 1) / FM) * ((p.N / 2 + 127) / 128);
    hipExtLaunchKernelGGL((nf4f_kernel<C_SWIGLU, 2>), dim3(tiles, 1, 1), dim3(256), 0, s, p.ev0,
                          p.ev1, 0, p);
    if (p.split_used) *p.split_used = 1;
    return hipGetLastError();
  }
  const Nf4fPlan plan = nf4f_plan(p.M, p.N, p.K);
  p.ksplit = plan.split;
  p.pstride = split_stride(p.M, p.N);
  if (p.ksplit > 1 && (!p.part || p.part_floats < p.ksplit * p.pstride)) p.ksplit = 1;
  if (plan.nt == 2) nf4f_launch_t<2>(p, s);
  else nf4f_launch_t<1>(p, s);
  if (p.split_used) *p.split_used = p.ksplit;
  if (p.ksplit > 1 && !p.defer_reduce) gemm_reduce_launch(p, s);
  return hipGetLastError();
}

}  // namespace lsn
