// bf16 MFMA GEMM for gfx950 with on-the-fly NF4 dequantization.
//
//   C[m, n] (op)= alpha * sum_k A(m, k) * B(n, k)   (+ LoRA extension, below)
//
// Both operands reach the matrix cores as bf16 with fp32 accumulation
// (v_mfma_f32_32x32x16_bf16).  Each operand comes through a loader that
// stages a 64-deep K slice into LDS, always k-contiguous per row, so the
// fragment reads are 16-byte ds_read_b128:
//   A_BF16_K  A(m,k) = A[m*lda + k]            (bf16, rows k-contiguous)
//   A_BF16_R  A(m,k) = A[k*lda + m]            (bf16, transposed storage)
//   A_F32_K   A(m,k) = bf16(A[m*lda + k])      (fp32 source rounded on load)
//   B_BF16_K  B(n,k) = B[n*ldb + k]
//   B_BF16_R  B(n,k) = B[k*ldb + n]
//   B_NF4_K   B(n,k) = bf16(level[code(e)] * absmax[e/64]),  e = n*rowlen + k
//   B_NF4_R   B(n,k) = same with e = k*rowlen + n   (transposed use, dX = dY W)
// NF4 codes are packed two per byte, even element in the low nibble; the
// dequantized value is the float32 product rounded once to bf16.
//
// The stored weight is W^T = [out, in] row-major, so the forward projection
// y = x W is (A_BF16_K, B_NF4_K) and the input gradient dx = dy W^T is
// (A_*_K, B_NF4_R).
//
// LoRA extension: with kext > 0 the reduction continues over kext extra
// columns taken straight from two bf16 matrices Aext [M, kext] and
// Bext [N, kext].  With Aext = bf16(s * x A) and Bext = B^T this adds
// s (x A) B inside the same accumulators (the low-rank branch of the
// adapted projection); several adapted projections that share one GEMM use a
// block layout (each projection's rows of Bext are zero outside its slot).
//
// Determinism: every output element is reduced by one lane in a fixed order,
// so results do not depend on scheduling, and they do not depend on where the
// weights live (a streamed slot or a resident record): the kernel only sees
// byte offsets inside the record.
#include "common.h"
#include <hip/hip_ext.h>

#include "gemm.h"
#include <type_traits>

namespace lsn {

constexpr int BK = 64;        // K depth staged per iteration
constexpr int PITCH = 72;     // LDS row pitch in bf16 (64 + 8 pad: conflict-free b128 reads)

// ---------------------------------------------------------------------------
// NF4 dequantization of one 32-bit code word (8 elements) to 4 packed bf16x2
// ---------------------------------------------------------------------------
LSN_DEV u32x4 nf4_dequant8(uint32_t w, float a, const float* lv) {
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float lo = lv[(w >> (8 * p)) & 15u] * a;
    const float hi = lv[(w >> (8 * p + 4)) & 15u] * a;
    r[p] = pack_bf16x2(lo, hi);
  }
  return r;
}

// ---------------------------------------------------------------------------
// operand loaders.  prefetch() issues the global loads of one 64-deep K slice
// into registers (no bounds checks when the slice is fully inside the
// matrix); store<Q>() converts / dequantizes the Q-th quarter of it and writes
// it to LDS as [row][k], so the four quarters can be interleaved with the four
// MFMA steps of the previous slice.
// ---------------------------------------------------------------------------
template <int CH, int Q>
struct Quarter {  // chunk indices i with 4*i/CH == Q
  static constexpr int lo = (Q * CH + 3) / 4, hi = ((Q + 1) * CH + 3) / 4;
};

// Addressing: init() computes each lane's 32-bit element offsets once; per
// slice only a uniform (scalar) base pointer moves, so a load is one
// scalar-base + vector-offset instruction.  Rows outside the matrix read
// row 0 and are zeroed; k beyond K (last slice only) likewise.
template <int ROWS, int NTHREADS>
struct LoadBf16K {  // rows k-contiguous bf16; base = &A(0, k0)
  static constexpr int CH = ROWS * 8 / NTHREADS;  // 16-byte chunks per thread
  u32x4 v[CH];
  uint32_t off[CH];
  uint32_t rowok;  // bit i: chunk i's row exists
  LSN_DEV void init(int64_t ld, int row0, int nrows) {
    rowok = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      const int row = row0 + (c >> 3), kc = (c & 7) * 8;
      const bool ok = row < nrows;
      rowok |= (ok ? 1u : 0u) << i;
      off[i] = (uint32_t)((ok ? (int64_t)row * ld : 0) + kc);
    }
  }
  LSN_DEV void prefetch(const uint16_t* base, int k0, int K, bool full) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int kc = ((threadIdx.x + i * NTHREADS) & 7) * 8;
      const bool ok = full || (((rowok >> i) & 1u) && k0 + kc < K);
      const u32x4 t = *reinterpret_cast<const u32x4*>(base + (ok ? off[i] : 0u));
      v[i] = ok ? t : u32x4{0, 0, 0, 0};
    }
  }
  template <int Q>
  LSN_DEV void store(uint16_t* lds) const {
#pragma unroll
    for (int i = Quarter<CH, Q>::lo; i < Quarter<CH, Q>::hi; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      *reinterpret_cast<u32x4*>(lds + (c >> 3) * PITCH + (c & 7) * 8) = v[i];
    }
  }
};

template <int ROWS, int NTHREADS>
struct LoadF32K {  // fp32 rows, rounded to bf16 on the way to LDS; base = &A(0, k0)
  static constexpr int CH = ROWS * 8 / NTHREADS;
  f32x4 v[CH][2];
  uint32_t off[CH];
  uint32_t rowok;
  LSN_DEV void init(int64_t ld, int row0, int nrows) {
    rowok = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      const int row = row0 + (c >> 3), kc = (c & 7) * 8;
      const bool ok = row < nrows;
      rowok |= (ok ? 1u : 0u) << i;
      off[i] = (uint32_t)((ok ? (int64_t)row * ld : 0) + kc);
    }
  }
  LSN_DEV void prefetch(const float* base, int k0, int K, bool full) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int kc = ((threadIdx.x + i * NTHREADS) & 7) * 8;
      const bool ok = full || (((rowok >> i) & 1u) && k0 + kc < K);
      const f32x4* p = reinterpret_cast<const f32x4*>(base + (ok ? off[i] : 0u));
      const f32x4 a0 = p[0], a1 = p[1];
      v[i][0] = ok ? a0 : f32x4{0, 0, 0, 0};
      v[i][1] = ok ? a1 : f32x4{0, 0, 0, 0};
    }
  }
  template <int Q>
  LSN_DEV void store(uint16_t* lds) const {
#pragma unroll
    for (int i = Quarter<CH, Q>::lo; i < Quarter<CH, Q>::hi; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      u32x4 o;
      o[0] = pack_bf16x2(v[i][0][0], v[i][0][1]);
      o[1] = pack_bf16x2(v[i][0][2], v[i][0][3]);
      o[2] = pack_bf16x2(v[i][1][0], v[i][1][1]);
      o[3] = pack_bf16x2(v[i][1][2], v[i][1][3]);
      *reinterpret_cast<u32x4*>(lds + (c >> 3) * PITCH + (c & 7) * 8) = o;
    }
  }
};

template <int ROWS, int NTHREADS>
struct LoadBf16R {  // element (row, k) at A[k*ld + row]; base = &A(k0 row of storage); 8x8 transpose
  static_assert(ROWS <= NTHREADS, "one 8x8 task per thread at most");
  u32x4 v[8];
  uint32_t off0;  // offset of (row group, k = kg*8)
  uint32_t ldu;
  bool rowok;
  LSN_DEV void init(int64_t ld, int row0, int nrows) {
    const int t = threadIdx.x;
    const int rg = (t >> 3), kg = t & 7;
    const int row = row0 + rg * 8;
    rowok = t < ROWS && row < nrows;
    off0 = (uint32_t)((int64_t)kg * 8 * ld + (rowok ? row : 0));
    ldu = (uint32_t)ld;
  }
  LSN_DEV void prefetch(const uint16_t* base, int k0, int K, bool full) {
    if (threadIdx.x >= ROWS) return;  // ROWS/8 row groups x 8 k groups
    const int kg = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = full || (rowok && k0 + kg * 8 + i < K);
      const u32x4 t = *reinterpret_cast<const u32x4*>(base + (ok ? off0 + (uint32_t)i * ldu : 0u));
      v[i] = ok ? t : u32x4{0, 0, 0, 0};
    }
  }
  template <int Q>
  LSN_DEV void store(uint16_t* lds) const {
    const int t = threadIdx.x;
    if (t >= ROWS) return;
    const int rg = t >> 3, kg = t & 7;
#pragma unroll
    for (int j = 2 * Q; j < 2 * Q + 2; ++j) {  // output row rg*8 + j holds k = kg*8 .. +7
      u32x4 o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t x = v[2 * p][j >> 1], y = v[2 * p + 1][j >> 1];
        o[p] = (j & 1) ? __builtin_amdgcn_perm(y, x, 0x07060302u)
                       : __builtin_amdgcn_perm(y, x, 0x05040100u);
      }
      *reinterpret_cast<u32x4*>(lds + (rg * 8 + j) * PITCH + kg * 8) = o;
    }
  }
};

template <int ROWS, int NTHREADS>
struct LoadNf4K {  // B(n,k) from W^T[n, k] (forward); one code word = 8 k
  static constexpr int CH = ROWS * 8 / NTHREADS;
  uint32_t code[CH];
  float amax[CH];
  uint32_t e[CH];  // element index of (row, kc) at k0 = 0
  uint32_t rowok;
  LSN_DEV void init(int64_t rowlen, int row0, int nrows) {
    rowok = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      const int row = row0 + (c >> 3), kc = (c & 7) * 8;
      const bool ok = row < nrows;
      rowok |= (ok ? 1u : 0u) << i;
      e[i] = (uint32_t)((ok ? (int64_t)row * rowlen : 0) + kc);
    }
  }
  // codes: byte base of the matrix; k0 even
  LSN_DEV void prefetch(const uint8_t* codes, const float* absmax, int k0, int K, bool full) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int kc = ((threadIdx.x + i * NTHREADS) & 7) * 8;
      const bool ok = full || (((rowok >> i) & 1u) && k0 + kc < K);
      const uint32_t ei = ok ? e[i] + (uint32_t)k0 : 0u;
      const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + (ei >> 1));
      const float am = absmax[ei >> 6];
      code[i] = ok ? cw : 0x77777777u;  // level 7 is exactly 0
      amax[i] = ok ? am : 0.f;
    }
  }
  template <int Q>
  LSN_DEV void store(uint16_t* lds, const float* lv) const {
#pragma unroll
    for (int i = Quarter<CH, Q>::lo; i < Quarter<CH, Q>::hi; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      *reinterpret_cast<u32x4*>(lds + (c >> 3) * PITCH + (c & 7) * 8) =
          nf4_dequant8(code[i], amax[i], lv);
    }
  }
};

template <int ROWS, int NTHREADS>
struct LoadNf4R {  // B(n,k) from W^T[k, n] (input gradient); task = KG k x 8 n
  // KG consecutive rows of W^T (k) by one code word (8 n) per thread, every
  // thread busy.  Lanes take consecutive k-groups, so a wave's KG*2-byte LDS
  // writes cover the banks evenly (conflict-free for KG = 2, two-way for 4).
  static constexpr int KG = 64 * ROWS / (8 * NTHREADS);
  static constexpr int NKG = 64 / KG;  // k-groups per slice
  static_assert(KG == 2 || KG == 4, "unsupported NF4 transpose tiling");
  uint32_t code[KG];
  float amax[KG];
  uint32_t e0;  // element index of (k = kg*KG, n) at k0 = 0
  uint32_t rl;
  bool rowok;
  LSN_DEV void init(int64_t rowlen, int row0, int nrows) {
    const int t = threadIdx.x;
    const int kg = t % NKG, ng = t / NKG;
    const int n = row0 + ng * 8;
    rowok = n < nrows;
    e0 = (uint32_t)((int64_t)kg * KG * rowlen + (rowok ? n : 0));
    rl = (uint32_t)rowlen;
  }
  LSN_DEV void prefetch(const uint8_t* codes, const float* absmax, int k0, int K, bool full) {
    const int kg = threadIdx.x % NKG;
    const uint32_t eb = e0 + (uint32_t)k0 * rl;
#pragma unroll
    for (int i = 0; i < KG; ++i) {
      const bool ok = full || (rowok && k0 + kg * KG + i < K);
      const uint32_t ei = ok ? eb + (uint32_t)i * rl : 0u;
      const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + (ei >> 1));
      const float am = absmax[ei >> 6];
      code[i] = ok ? cw : 0x77777777u;
      amax[i] = ok ? am : 0.f;
    }
  }
  template <int Q>
  LSN_DEV void store(uint16_t* lds, const float* lv) const {
    const int t = threadIdx.x;
    const int kg = t % NKG, ng = t / NKG;
#pragma unroll
    for (int j = 2 * Q; j < 2 * Q + 2; ++j) {  // LDS row n = ng*8 + j, k = kg*KG ..
      if constexpr (KG == 4) {
        u32x2 o;
        o[0] = pack_bf16x2(lv[(code[0] >> (4 * j)) & 15u] * amax[0],
                           lv[(code[1] >> (4 * j)) & 15u] * amax[1]);
        o[1] = pack_bf16x2(lv[(code[2] >> (4 * j)) & 15u] * amax[2],
                           lv[(code[3] >> (4 * j)) & 15u] * amax[3]);
        *reinterpret_cast<u32x2*>(lds + (ng * 8 + j) * PITCH + kg * 4) = o;
      } else {
        *reinterpret_cast<uint32_t*>(lds + (ng * 8 + j) * PITCH + kg * 2) =
            pack_bf16x2(lv[(code[0] >> (4 * j)) & 15u] * amax[0],
                        lv[(code[1] >> (4 * j)) & 15u] * amax[1]);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// kernel
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN, int NS, int OPA, int OPB>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_kernel(const GemmParams p) {
  static_assert(NS % 2 == 0, "register stages come in pairs (two LDS buffers)");
  constexpr int NTHREADS = WGM * WGN * 64;   // waves arranged WGM x WGN
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1, "tile too small");
  constexpr bool NF4B = (OPB == B_NF4_K || OPB == B_NF4_R);

  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * PITCH];
  __shared__ float sLv[16];

  // ---- tile coordinates (XCD-aware: consecutive ids land on one XCD) ----
  const int mt = (p.M + BM - 1) / BM;
  const int nblk = gridDim.x, b = blockIdx.x;
  const int per = nblk / 8, rem = nblk % 8, x = b % 8;
  const int id = x * per + min(x, rem) + b / 8;
  const int m0 = (id % mt) * BM, n0 = (id / mt) * BN;
  if (p.causal == CAUSAL_SKIP_UPPER && n0 >= m0 + BM) return;  // uniform per workgroup

  const int z = blockIdx.z;
  const int zo = z / p.zdiv, zi = z % p.zdiv;
  const int64_t offA = zo * p.sA_o + zi * p.sA_i;
  const int64_t offB = zo * p.sB_o + (zi / p.grpB) * p.sB_i;
  const int64_t offC = zo * p.sC_o + zi * p.sC_i;

  if (threadIdx.x < 16) sLv[threadIdx.x] = p.levels[threadIdx.x];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // loaders: NS register stages (slices it+1 .. it+NS while slice it computes)
  using LA = typename std::conditional<
      OPA == A_BF16_K, LoadBf16K<BM, NTHREADS>,
      typename std::conditional<OPA == A_F32_K, LoadF32K<BM, NTHREADS>,
                                LoadBf16R<BM, NTHREADS>>::type>::type;
  using LB = typename std::conditional<
      OPB == B_BF16_K, LoadBf16K<BN, NTHREADS>,
      typename std::conditional<
          OPB == B_BF16_R, LoadBf16R<BN, NTHREADS>,
          typename std::conditional<OPB == B_NF4_K, LoadNf4K<BN, NTHREADS>,
                                    LoadNf4R<BN, NTHREADS>>::type>::type>::type;
  LA la[NS];
  LB lb[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    la[q].init(p.lda, m0, p.M);
    if constexpr (NF4B)
      lb[q].init(p.rowlen, n0, p.N);
    else
      lb[q].init(p.ldb, n0, p.N);
  }

  const int nkt = (p.K + BK - 1) / BK;
  // k-tiles [kt_lo, kt_lo + nk) of every segment (all of them unless causal)
  int kt_lo = 0, nk = nkt;
  if (p.causal == CAUSAL_K_TO_ROW) nk = min(nkt, (m0 + BM + BK - 1) / BK);
  if (p.causal == CAUSAL_K_FROM_ROW) {
    kt_lo = min(nkt, m0 / BK);
    nk = nkt - kt_lo;
  }
  // split-k: blockIdx.y takes tiles [it0, it1) of the nseg * nk
  const int ntile = nk * p.nseg;
  const int kper = (ntile + p.ksplit - 1) / p.ksplit;
  const int it0 = min(ntile, (int)blockIdx.y * kper), it1 = min(ntile, it0 + kper);
  const bool rows_a_full = m0 + BM <= p.M, rows_b_full = n0 + BN <= p.N;

  // uniform per-slice base pointers; per-lane offsets were fixed by init()
  auto prefetch = [&](LA& a, LB& bb, int it) {
    const int seg = it / max(nk, 1), k0 = (kt_lo + it % max(nk, 1)) * BK;
    const bool kfull = k0 + BK <= p.K;
    const int64_t ka = (OPA == A_BF16_R) ? (int64_t)k0 * p.lda : k0;
    if constexpr (OPA == A_F32_K)
      a.prefetch(reinterpret_cast<const float*>(p.A) + offA + seg * p.sA_seg + ka, k0, p.K,
                 rows_a_full && kfull);
    else
      a.prefetch(reinterpret_cast<const uint16_t*>(p.A) + offA + seg * p.sA_seg + ka, k0, p.K,
                 rows_a_full && kfull);
    if constexpr (NF4B) {
      bb.prefetch(reinterpret_cast<const uint8_t*>(p.B), p.absmax, k0, p.K, rows_b_full && kfull);
    } else {
      const int64_t kb = (OPB == B_BF16_R) ? (int64_t)k0 * p.ldb : k0;
      bb.prefetch(reinterpret_cast<const uint16_t*>(p.B) + offB + seg * p.sB_seg + kb, k0, p.K,
                  rows_b_full && kfull);
    }
  };
  auto store_q = [&](auto q_, const LA& a, const LB& bb, int buf) {
    constexpr int Q = decltype(q_)::value;
    a.template store<Q>(sA[buf]);
    if constexpr (NF4B)
      bb.template store<Q>(sB[buf], sLv);
    else
      bb.template store<Q>(sB[buf]);
  };

  const int lr = lane & 31, lk = (lane >> 5) * 8;
  // One K slice: slice it sits in LDS buffer S & 1 (stage S held it); the
  // next slice (stage S+1) is stored, in quarters between the MFMA steps,
  // into the other buffer, and stage S is refilled with slice it+NS.
  // Fragments are double buffered: step KK+1's LDS reads are issued before
  // step KK's MFMAs.
  auto body = [&](auto s_, int it) {
    constexpr int S = decltype(s_)::value;
    constexpr int B = S & 1, SN = (S + 1) % NS;
    // Unconditional (branch-free body): past the end the prefetch re-reads the
    // last slice and the store fills a buffer no one reads any more.
    prefetch(la[S], lb[S], min(it + NS, it1 - 1));
    const uint16_t* a_base = sA[B] + (wm * WTM + lr) * PITCH + lk;
    const uint16_t* b_base = sB[B] + (wn * WTN + lr) * PITCH + lk;
    bf16x8 af[2][TM], bfr[2][TN];
    auto read = [&](int f, int kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[f][i] = *reinterpret_cast<const bf16x8*>(a_base + i * 32 * PITCH + kk * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[f][j] = *reinterpret_cast<const bf16x8*>(b_base + j * 32 * PITCH + kk * 16);
    };
    auto kstep = [&](auto kk_) {
      constexpr int KK = decltype(kk_)::value;
      if constexpr (KK < BK / 16 - 1) read((KK + 1) & 1, KK + 1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[KK & 1][i], bfr[KK & 1][j],
                                                               acc[i][j], 0, 0, 0);
      store_q(std::integral_constant<int, KK>{}, la[SN], lb[SN], B ^ 1);
    };
    read(0, 0);
    kstep(std::integral_constant<int, 0>{});
    kstep(std::integral_constant<int, 1>{});
    kstep(std::integral_constant<int, 2>{});
    kstep(std::integral_constant<int, 3>{});
    __syncthreads();
  };

  if (it1 > it0) {
#pragma unroll
    for (int q = 0; q < NS; ++q) prefetch(la[q], lb[q], min(it0 + q, it1 - 1));
    __syncthreads();  // sLv visible
    store_q(std::integral_constant<int, 0>{}, la[0], lb[0], 0);
    store_q(std::integral_constant<int, 1>{}, la[0], lb[0], 0);
    store_q(std::integral_constant<int, 2>{}, la[0], lb[0], 0);
    store_q(std::integral_constant<int, 3>{}, la[0], lb[0], 0);
    __syncthreads();
    // stage (it - it0) % NS holds slice it; its LDS buffer is that parity
    for (int it = it0; it < it1; it += NS) {
      body(std::integral_constant<int, 0>{}, it);
      if (it + 1 < it1) body(std::integral_constant<int, 1>{}, it + 1);
      if constexpr (NS > 2) {
        if (it + 2 < it1) body(std::integral_constant<int, 2 % NS>{}, it + 2);
        if (it + 3 < it1) body(std::integral_constant<int, 3 % NS>{}, it + 3);
      }
    }
  }

  // ---- LoRA extension: extra k columns read directly as fragments ----
  if (p.kext > 0 && blockIdx.y == 0) {
    for (int e0 = 0; e0 < p.kext; e0 += 16) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = m0 + wm * WTM + i * 32 + lr;
        if (m < p.M)
          af[i] = *reinterpret_cast<const bf16x8*>(p.Aext + (int64_t)m * p.ldae + e0 + lk);
        else
          af[i] = bf16x8{};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WTN + j * 32 + lr;
        if (n < p.N)
          bfr[j] = *reinterpret_cast<const bf16x8*>(p.Bext + (int64_t)n * p.ldbe + e0 + lk);
        else
          bfr[j] = bf16x8{};
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: lane holds column lr, rows (e/4)*8 + (lane/32)*4 + e%4 ----
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * WTN + j * 32 + lr;
      if (n >= p.N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * WTM + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (m >= p.M) continue;
        if (p.ksplit > 1) {  // raw partial sum of this k range
          p.part[blockIdx.y * p.pstride + (int64_t)m * p.N + n] = acc[i][j][e];
          continue;
        }
        const float v = p.alpha * acc[i][j][e];
        const int64_t o = offC + (int64_t)m * p.ldc + n;
        switch (p.cmode) {
          case C_F32: reinterpret_cast<float*>(p.C)[o] = v; break;
          case C_F32_ACC: reinterpret_cast<float*>(p.C)[o] += v; break;
          case C_F32_RES:
            reinterpret_cast<float*>(p.C)[o] = p.R[offC + (int64_t)m * p.ldr + n] + v;
            break;
          default: reinterpret_cast<uint16_t*>(p.C)[o] = f32_to_bf16_bits(v); break;
        }
      }
    }
}

// ---------------------------------------------------------------------------
// split-k reduction: partial sums added in split order, then the epilogue
// ---------------------------------------------------------------------------
__global__ void gemm_reduce_k(const GemmParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)p.M * p.N) return;
  const int m = (int)(i / p.N), n = (int)(i % p.N);
  float acc = 0.f;
  for (int y = 0; y < p.ksplit; ++y) acc += p.part[y * p.pstride + (int64_t)m * p.N + n];
  const float v = p.alpha * acc;
  const int64_t o = (int64_t)m * p.ldc + n;
  switch (p.cmode) {
    case C_F32: reinterpret_cast<float*>(p.C)[o] = v; break;
    case C_F32_ACC: reinterpret_cast<float*>(p.C)[o] += v; break;
    case C_F32_RES: reinterpret_cast<float*>(p.C)[o] = p.R[(int64_t)m * p.ldr + n] + v; break;
    default: reinterpret_cast<uint16_t*>(p.C)[o] = f32_to_bf16_bits(v); break;
  }
}

// The same reduction, four columns per thread and one block row per output
// row (blockIdx.y = m): four splits are loaded at a time and then added in
// split order, as above, so results are bitwise the same.  Needs N % 4 == 0
// and 16-byte aligned rows.
template <int CM>
__global__ void gemm_reduce4_k(const GemmParams p) {
  const int m = blockIdx.y;
  const int n = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (n >= p.N) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(p.part + (int64_t)m * p.N + n);
  const int64_t stride = p.pstride / 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int y = 0;
  for (; y + 4 <= p.ksplit; y += 4) {
    const f32x4 a = src[y * stride], b = src[(y + 1) * stride];
    const f32x4 c = src[(y + 2) * stride], d = src[(y + 3) * stride];
    acc += a;
    acc += b;
    acc += c;
    acc += d;
  }
  for (; y < p.ksplit; ++y) acc += src[y * stride];
  const f32x4 r = p.alpha * acc;
  const int64_t o = (int64_t)m * p.ldc + n;
  if constexpr (CM == C_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.C) + o) = r;
  } else if constexpr (CM == C_F32_ACC) {
    f32x4* c = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.C) + o);
    *c = *c + r;
  } else if constexpr (CM == C_F32_RES) {
    const f32x4 res = *reinterpret_cast<const f32x4*>(p.R + (int64_t)m * p.ldr + n);
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.C) + o) = res + r;
  } else {
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.C) + o) =
        u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
  }
}

void gemm_reduce_launch(const GemmParams& p, hipStream_t s) {
  const bool bf = p.cmode == C_BF16;
  const bool vec = p.M <= 65535 && p.N % 4 == 0 && p.pstride % 4 == 0 && p.ldc % 4 == 0 &&
                   ((uintptr_t)p.part & 15) == 0 && ((uintptr_t)p.C & (bf ? 7 : 15)) == 0 &&
                   (p.cmode != C_F32_RES || (p.ldr % 4 == 0 && ((uintptr_t)p.R & 15) == 0));
  if (!vec) {
    const int64_t n = (int64_t)p.M * p.N;
    hipLaunchKernelGGL(gemm_reduce_k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
    return;
  }
  const dim3 grid((unsigned)((p.N / 4 + 255) / 256), (unsigned)p.M);
  if (p.cmode == C_F32) hipLaunchKernelGGL(gemm_reduce4_k<C_F32>, grid, dim3(256), 0, s, p);
  else if (p.cmode == C_F32_ACC) hipLaunchKernelGGL(gemm_reduce4_k<C_F32_ACC>, grid, dim3(256), 0, s, p);
  else if (p.cmode == C_F32_RES) hipLaunchKernelGGL(gemm_reduce4_k<C_F32_RES>, grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL(gemm_reduce4_k<C_BF16>, grid, dim3(256), 0, s, p);
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------
// Tile and split-k choice.  M >= 256 takes the 256 x 128 tile (each
// dequantized weight feeds 256 rows).  A single problem with fewer than 200
// tiles splits its k range so that about 256 workgroups run (one per CU);
// batched problems choose smaller tiles instead.
GemmPlan gemm_plan(int M, int N, int K, int nseg, int batch) {
  GemmPlan g;
  const int64_t t256 = (int64_t)((M + 255) / 256) * ((N + 127) / 128) * batch;
  const int64_t t128 = (int64_t)((M + 127) / 128) * ((N + 127) / 128) * batch;
  const int64_t t64 = (int64_t)((M + 63) / 64) * ((N + 63) / 64) * batch;
  int64_t tiles;
  if (batch == 1) {
    if (M >= 256) { g.tile = TILE_256x128; tiles = t256; }
    else if (M >= 128) { g.tile = TILE_128x128; tiles = t128; }
    else { g.tile = TILE_64x64; tiles = t64; }
    const int nkt = (K + 63) / 64 * nseg;
    if (tiles > 0 && tiles < 200) {  // (no tiles at M = 0: nothing to split)
      int sp = (int)std::min<int64_t>(8, (256 + tiles - 1) / tiles);
      sp = std::min(sp, std::max(1, nkt / 4));
      g.split = std::max(sp, 1);
    }
  } else {
    // (the attention products, 32 heads of 512 x 128: 64 x 64, 512 workgroups,
    // measured 20-23 us against 28-32 us on 128 x 128)
    if (M >= 256 && t256 >= 192) g.tile = TILE_256x128;
    else if (M >= 128 && t128 >= 512) g.tile = TILE_128x128;
    else g.tile = TILE_64x64;
  }
  return g;
}

int64_t gemm_partial_floats(int M, int N, int K, int nseg, int batch) {
  const GemmPlan g = gemm_plan(M, N, K, nseg, batch);
  int64_t f = g.split > 1 ? g.split * split_stride(M, N) : 0;
  if (batch == 1 && nseg == 1 && M >= 256 && K % 64 == 0) {  // the fused NF4 kernels
    const int sp = std::max(nf4f_split(M, N, K), nf4f_plan(M, N, K).split);
    if (sp > 1) f = std::max<int64_t>(f, sp * split_stride(M, N));
  }
  return f;
}

int gemm_tile(const GemmParams& p, int opa, int opb, int batch) {
  if (opa == A_BF16_K && opb == B_NF4_K && nf4f_eligible(p, batch)) return TILE_NF4F;
  if (opa == A_BF16_K && opb == B_NF4_R && nf4t_eligible(p, batch)) return TILE_NF4T;
  if (opa == A_BF16_K && opb == B_BF16_K && bf16f_eligible(p, batch)) return TILE_BF16F;
  if (opa == A_BF16_K && opb == B_BF16_R && bf16t_eligible(p, batch)) return TILE_BF16T;
  return gemm_plan(p.M, p.N, p.K, p.nseg, batch).tile;
}

template <int BM, int BN, int WGM, int WGN, int NS, int OPA, int OPB>
static hipError_t launch_t(const GemmParams& p, int batch, hipStream_t s) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  // the timing events, when given, ride on the kernel's own dispatch (no
  // extra packets around it)
  hipExtLaunchKernelGGL((gemm_kernel<BM, BN, WGM, WGN, NS, OPA, OPB>), dim3(tiles, p.ksplit, batch),
                        dim3(WGM * WGN * 64), 0, s, p.ev0, p.ev1, 0, p);
  if (p.split_used) *p.split_used = p.ksplit;
  if (p.ksplit > 1 && !p.defer_reduce) gemm_reduce_launch(p, s);
  return hipGetLastError();
}

template <int OPA, int OPB>
static hipError_t launch_tiles(GemmParams p, int batch, hipStream_t s) {
  const GemmPlan g = gemm_plan(p.M, p.N, p.K, p.nseg, batch);
  p.ksplit = g.split;
  p.pstride = split_stride(p.M, p.N);
  if (p.ksplit > 1 && (!p.part || p.part_floats < p.ksplit * p.pstride)) p.ksplit = 1;
  switch (g.tile) {
    // 256 x 128: 8 waves (two per SIMD) of 64 x 64; smaller tiles: 4 waves
    case TILE_256x128: return launch_t<256, 128, 4, 2, 2, OPA, OPB>(p, batch, s);
    case TILE_128x128: return launch_t<128, 128, 2, 2, 2, OPA, OPB>(p, batch, s);
    default: return launch_t<64, 64, 2, 2, 2, OPA, OPB>(p, batch, s);
  }
}

// The loaders address within one matrix (one batch entry and segment) with
// 32-bit element offsets; larger matrices are rejected.
static bool offsets_fit(const GemmParams& p, int opa, int opb) {
  const int64_t lim = (int64_t)1 << 31;
  const int64_t a_ext = (opa == A_BF16_R) ? (int64_t)p.K * p.lda + p.M : (int64_t)p.M * p.lda + p.K;
  int64_t b_ext;
  if (opb == B_NF4_K) b_ext = (int64_t)p.N * p.rowlen + p.K;
  else if (opb == B_NF4_R) b_ext = (int64_t)p.K * p.rowlen + p.N;
  else if (opb == B_BF16_R) b_ext = (int64_t)p.K * p.ldb + p.N;
  else b_ext = (int64_t)p.N * p.ldb + p.K;
  return a_ext < lim && b_ext < lim;
}

hipError_t gemm(const GemmParams& p, int opa, int opb, int batch, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0 || batch <= 0) return hipSuccess;
  if (!offsets_fit(p, opa, opb)) return hipErrorInvalidValue;
  if (p.cmode == C_SWIGLU)  // the forward NF4 kernel's epilogue only
    return opa == A_BF16_K && opb == B_NF4_K && batch == 1 ? nf4f_launch(p, s) : hipErrorInvalidValue;
  if (opa == A_BF16_K && opb == B_NF4_K && nf4f_eligible(p, batch)) return nf4f_launch(p, s);
  if (opa == A_BF16_K && opb == B_NF4_R && nf4t_eligible(p, batch)) return nf4t_launch(p, s);
  if (opa == A_BF16_K && opb == B_BF16_K && bf16f_eligible(p, batch)) return bf16f_launch(p, s);
  if (opa == A_BF16_K && opb == B_BF16_R && bf16t_eligible(p, batch)) return bf16t_launch(p, s);
#define LSN_CASE(A_, B_) \
  if (opa == A_ && opb == B_) return launch_tiles<A_, B_>(p, batch, s);
  LSN_CASE(A_BF16_K, B_NF4_K)
  LSN_CASE(A_BF16_K, B_NF4_R)
  LSN_CASE(A_F32_K, B_NF4_R)
  LSN_CASE(A_BF16_K, B_BF16_K)
  LSN_CASE(A_BF16_K, B_BF16_R)
  LSN_CASE(A_BF16_R, B_BF16_R)
#undef LSN_CASE
  return hipErrorInvalidValue;
}

}  // namespace lsn
