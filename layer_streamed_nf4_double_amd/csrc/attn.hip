// Causal grouped-query attention in one kernel per layer pass, forward and
// the query side of the backward:
//
//   forward:   S = alpha q k^T (keys <= query), P = softmax(S) over the row,
//              O = P v
//   backward:  dP = dO v^T, dS = P (dP - rowsum(P dP)), dQ = alpha dS k
//
// One workgroup (eight waves) per (sequence, q head, 64-query tile).  The
// tile's 64 x (q0 + 64) score (or dP) rows live in LDS (fp32, at most 129
// KiB), so they never round-trip through HBM; the forward writes only O
// (bf16) and, in the backward's recompute, the probabilities the backward
// reads (P in fp32, P in bf16 for dV); the backward writes dS (bf16, for dK)
// and dQ (fp32).  Both run the same three phases:
//
// Phase 1 (scores / dP): MFMA v_mfma_f32_32x32x16_bf16 with the keys as the
// first operand (k, or v for dP) and the queries as the second (q, or dO),
// so a lane's accumulators are four consecutive keys of one query row: one
// 16-byte LDS store each.  Wave w takes the 32-key tiles j = w, w + 8, ...
// of the tile's causal extent.
// Phase 2: 16 lanes per row, a wave takes four rows at a time.  Forward: the
// arithmetic of a two-pass softmax (max and sum over keys <= query, one exp
// per element).  Backward: D = sum over keys <= query of P dP, then
// dS = P (dP - D).  The bf16 result (P or dS) overwrites the front half of
// the row.
// Phase 3 (O^T = v^T P^T, or dQ^T = k^T dS^T): the first operand is v^T (k^T)
// (an MFMA operand needs 8 consecutive keys per lane), the second is P (dS)
// from LDS; a lane's accumulators are four consecutive head dimensions of
// one query: one store each.
//
// Operand layout.  A fragment of q, k, v, dO or their transposes is 64 lanes
// x 16 bytes taken from 32 rows; read from the row-major rows, every load
// instruction would touch 32 rows.  attn_prep_k first writes
// fragment-ordered copies (each fragment 1 KiB contiguous, lane-major), so
// every operand load of the fused kernel is one contiguous 1 KiB per wave.
//
// Every output is written by one lane after a fixed-order reduction:
// results are deterministic, and the forward's are the same with or without
// the P outputs.
#include "common.h"

#include "attn.h"

namespace lsn {

namespace {
constexpr int QT = 64;          // queries per workgroup
constexpr int NW = 8;           // waves per workgroup (two per SIMD)
constexpr int SMAX = 512;       // longest sequence the LDS score tile holds
constexpr int RS = SMAX + 4;    // LDS row stride (floats): rows 4 banks apart

// reductions over the 16 lanes of a row group, fixed butterfly order
LSN_DEV float row16_max(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
LSN_DEV float row16_sum(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Fragment regions (attn_prep_k): region 0, the nq query-side heads as row
// fragments (q or dO); region 1, the nkv key-side heads as row fragments (k,
// or v for dP); region 2, the nkv heads as transposed fragments (v^T, or
// k^T for dQ).  512 elements per fragment.
struct AttnK {
  const uint16_t* frag;
  const float* Pin;    // backward: P (fp32, rows of S)
  float* Pf;           // forward: P out (fp32), or null
  uint16_t* Pb;        // forward: P out (bf16), or null; backward: dS out
  uint16_t* O;         // forward output
  int64_t ldo;
  float* dQ;           // backward output
  int64_t ldq;
  int n_seq, S, nq, nkv;
  float alpha;
};

// region r's head slot h takes columns col + h d of rows ld apart
struct PrepSrc {
  const uint16_t* p;
  int64_t ld, col;
};
}  // namespace

template <int D, bool BWD>
__global__ __launch_bounds__(64 * NW) void attn_k(const AttnK p) {
  constexpr int KS = D / 16;  // MFMA k-steps over the head dimension
  __shared__ __attribute__((aligned(16))) float sS[QT * RS];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  const int S = p.S, nq = p.nq;
  const int qt = blockIdx.x, z = blockIdx.y;
  const int seq = z / nq, h = z % nq, kvh = h / (nq / p.nkv);
  const int q0 = qt * QT, nk = q0 + QT;  // keys 0 .. nk - 1
  const int nt32 = S / 32;
  const uint16_t* F0 = p.frag + ((int64_t)(seq * nq + h) * nt32 + q0 / 32) * KS * 512 + lane * 8;
  const uint16_t* F1 = p.frag + (int64_t)p.n_seq * S * nq * D +
                       (int64_t)(seq * p.nkv + kvh) * nt32 * KS * 512 + lane * 8;

  // ---- phase 1: the tile's 64 query rows against keys < nk ----
  // key tiles j = w, w + NW, ...: key fragments double buffered (ka: j, kb: j + NW)
  const int nkt = nk / 32;
  {
    bf16x8 qf[2][KS], ka[KS], kb[KS];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        qf[i][kk] = *reinterpret_cast<const bf16x8*>(F0 + (i * KS + kk) * 512);
    auto load_k = [&](bf16x8 (&f)[KS], int j) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) f[kk] = *reinterpret_cast<const bf16x8*>(F1 + (j * KS + kk) * 512);
    };
    const float scale = BWD ? 1.0f : p.alpha;  // scores alpha q k^T; dP unscaled
    auto tile = [&](const bf16x8 (&f)[KS], int j) {
      f32x16 acc[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[kk], qf[i][kk], acc[i], 0, 0, 0);
      // acc[i][4 g + t]: query 32 i + lr, key 32 j + 8 g + 4 hh + t
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = {scale * acc[i][4 * g], scale * acc[i][4 * g + 1],
                           scale * acc[i][4 * g + 2], scale * acc[i][4 * g + 3]};
          *reinterpret_cast<f32x4*>(&sS[(32 * i + lr) * RS + 32 * j + 8 * g + 4 * hh]) = v;
        }
    };
    if (w < nkt) load_k(ka, w);
    if (w + NW < nkt) load_k(kb, w + NW);
    for (int j = w; j < nkt; j += 2 * NW) {
      tile(ka, j);
      if (j + 2 * NW < nkt) load_k(ka, j + 2 * NW);
      if (j + NW < nkt) {
        tile(kb, j + NW);
        if (j + 3 * NW < nkt) load_k(kb, j + 3 * NW);
      }
    }
  }
  // phase 3's first transposed fragments (one (head-dimension tile, query
  // tile) pair per wave; with d = 64 only four waves have one; chunks of 64
  // keys, double buffered), loaded now so that they arrive during phase 2
  constexpr int NDT = D / 32;  // 32-wide head-dimension tiles
  const int dt = w % NDT, qi = w / NDT;
  const bool pv_wave = qi < 2;
  const int nch = nk / 64;     // 64-key chunks of the tile's extent
  const uint16_t* F2 = p.frag + (int64_t)p.n_seq * S * (nq + p.nkv) * D +
                       ((int64_t)(seq * p.nkv + kvh) * NDT + dt) * (S / 16) * 512 + lane * 8;
  bf16x8 va[4], vb[4];
  auto load_v = [&](bf16x8 (&f)[4], int ch) {  // k-steps 4 ch .. 4 ch + 3
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) f[kk] = *reinterpret_cast<const bf16x8*>(F2 + (4 * ch + kk) * 512);
  };
  if (pv_wave) {
    load_v(va, 0);
    if (nch > 1) load_v(vb, 1);
  }
  __syncthreads();

  // ---- phase 2: lane s of a row takes its 16-byte chunks s, s + 16, ... ----
  {
    const int sub = lane & 15;
#pragma unroll 1
    for (int rnd = 0; rnd < QT / (4 * NW); ++rnd) {
      const int r = rnd * 4 * NW + w * 4 + (lane >> 4), i = q0 + r;  // i: query position
      float* row = &sS[r * RS];
      const int64_t prow = ((int64_t)z * S + i) * S;  // row i of head z in Pf / Pb
      f32x4 v[SMAX / 64];
      if constexpr (!BWD) {  // softmax
        float m = -INFINITY;
#pragma unroll
        for (int u = 0; u < SMAX / 64; ++u) {
          const int c = sub + 16 * u;
          v[u] = 4 * c < nk ? *reinterpret_cast<const f32x4*>(row + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * c + e <= i) m = fmaxf(m, v[u][e]);
        }
        m = row16_max(m);
        float sum = 0.f;
#pragma unroll
        for (int u = 0; u < SMAX / 64; ++u) {
          const int c = sub + 16 * u;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ex = 4 * c + e <= i ? expf(v[u][e] - m) : 0.f;
            v[u][e] = ex;
            sum += ex;
          }
        }
        sum = row16_sum(sum);
        const float inv = 1.0f / sum;
#pragma unroll
        for (int u = 0; u < SMAX / 64; ++u) v[u] = v[u] * inv;
      } else {  // dS = P (dP - sum over keys <= query of P dP)
        f32x4 pv[SMAX / 64];
        float dot = 0.f;
#pragma unroll
        for (int u = 0; u < SMAX / 64; ++u) {
          const int c = sub + 16 * u;
          const bool in = 4 * c < nk;
          v[u] = in ? *reinterpret_cast<const f32x4*>(row + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
          pv[u] = in ? *reinterpret_cast<const f32x4*>(p.Pin + prow + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * c + e <= i) dot += pv[u][e] * v[u][e];
        }
        dot = row16_sum(dot);
#pragma unroll
        for (int u = 0; u < SMAX / 64; ++u) {
          const int c = sub + 16 * u;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[u][e] = 4 * c + e <= i ? pv[u][e] * (v[u][e] - dot) : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < SMAX / 64; ++u) {
        const int c = sub + 16 * u;
        if (4 * c >= nk) continue;
        const u32x2 pb = {pack_bf16x2(v[u][0], v[u][1]), pack_bf16x2(v[u][2], v[u][3])};
        // bf16 over the front half of the row: the row's 16 lanes are in one
        // wave, and all their reads precede (through the row sums) any write
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(row) + 4 * c) = pb;
        if (!BWD && p.Pf) *reinterpret_cast<f32x4*>(p.Pf + prow + 4 * c) = v[u];
        if (p.Pb) *reinterpret_cast<u32x2*>(p.Pb + prow + 4 * c) = pb;
      }
      if (p.Pb)  // keys beyond the tile's extent: zero
        for (int c = nk / 4 + sub; c < S / 4; c += 16)
          *reinterpret_cast<u32x2*>(p.Pb + prow + 4 * c) = u32x2{0u, 0u};
    }
  }
  __syncthreads();

  // ---- phase 3: O^T[d][q] = sum over keys of v^T[d][key] P^T[key][q]
  // (backward: dQ^T = alpha k^T dS^T) ----
  {
    if (!pv_wave) return;
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    const char* sP = reinterpret_cast<const char*>(sS) + (32 * qi + lr) * RS * 4 + 16 * hh;
    // every k-step of the tile's extent: P (dS) is zero for keys beyond a query
    auto pv = [&](const bf16x8 (&f)[4], int ch) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 pf = *reinterpret_cast<const bf16x8*>(sP + (64 * ch + 16 * kk) * 2);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[kk], pf, acc, 0, 0, 0);
      }
    };
    for (int ch = 0; ch < nch; ch += 2) {
      pv(va, ch);
      if (ch + 2 < nch) load_v(va, ch + 2);
      if (ch + 1 < nch) {
        pv(vb, ch + 1);
        if (ch + 3 < nch) load_v(vb, ch + 3);
      }
    }
    // acc[4 g + t]: head dimension dt 32 + 8 g + 4 hh + t, query 32 qi + lr
    const int64_t t = (int64_t)seq * S + q0 + 32 * qi + lr;
    if constexpr (!BWD) {
      uint16_t* o = p.O + t * p.ldo + h * D + dt * 32 + 4 * hh;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<u32x2*>(o + 8 * g) = u32x2{pack_bf16x2(acc[4 * g], acc[4 * g + 1]),
                                                     pack_bf16x2(acc[4 * g + 2], acc[4 * g + 3])};
    } else {
      float* o = p.dQ + t * p.ldq + h * D + dt * 32 + 4 * hh;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(o + 8 * g) =
            f32x4{p.alpha * acc[4 * g], p.alpha * acc[4 * g + 1], p.alpha * acc[4 * g + 2],
                  p.alpha * acc[4 * g + 3]};
    }
  }
}

// Fragment-ordered copies for attn_k, one 32-token x d slab of one head per
// block (blockIdx.z: region 0's nq heads, then region 1's nkv heads, then
// region 2's nkv heads).  Row fragments (tile t, k-step kk): lane
// l = 32 hh + lr holds row 32 t + lr, dimensions 16 kk + 8 hh .. +7.
// Transposed fragments (dimension tile dt, key step ks): lane l holds
// dimension 32 dt + lr, rows 16 ks + 8 hh .. +7 (through an LDS transpose).
// Writes are 16 bytes per lane, contiguous.
template <int D>
__global__ __launch_bounds__(256) void attn_prep_k(const PrepSrc s0, const PrepSrc s1,
                                                   const PrepSrc s2, int S, int n_seq, int nq,
                                                   int nkv, uint16_t* __restrict__ frag) {
  constexpr int KS = D / 16;
  __shared__ uint16_t t[D][32 + 8];
  const int t32 = blockIdx.x, seq = blockIdx.y, hs = blockIdx.z;
  const int nt32 = S / 32;
  if (hs < nq + nkv) {  // row fragments: a permutation of 16-byte chunks
    const bool r0 = hs < nq;
    const int hd = r0 ? hs : hs - nq;
    const PrepSrc& sr = r0 ? s0 : s1;
    const uint16_t* src = sr.p + ((int64_t)seq * S + 32 * t32) * sr.ld + sr.col + (int64_t)hd * D;
    const int64_t base = r0 ? ((int64_t)(seq * nq + hd) * nt32 + t32) * KS * 512
                            : (int64_t)n_seq * S * nq * D +
                                  ((int64_t)(seq * nkv + hd) * nt32 + t32) * KS * 512;
    for (int c = threadIdx.x; c < KS * 64; c += 256) {
      const int kk = c >> 6, l = c & 63;
      const u32x4 x = *reinterpret_cast<const u32x4*>(src + (int64_t)(l & 31) * sr.ld + 16 * kk + 8 * (l >> 5));
      *reinterpret_cast<u32x4*>(frag + base + (int64_t)c * 8) = x;
    }
    return;
  }
  const int kv = hs - nq - nkv;
  const uint16_t* src = s2.p + ((int64_t)seq * S + 32 * t32) * s2.ld + s2.col + (int64_t)kv * D;
  for (int c = threadIdx.x; c < 32 * D / 8; c += 256) {
    const int tok = c / (D / 8), j0 = (c % (D / 8)) * 8;
    const u32x4 x = *reinterpret_cast<const u32x4*>(src + (int64_t)tok * s2.ld + j0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t[j0 + 2 * e][tok] = (uint16_t)(x[e] & 0xFFFFu);
      t[j0 + 2 * e + 1][tok] = (uint16_t)(x[e] >> 16);
    }
  }
  __syncthreads();
  // this slab holds key steps 2 t32 and 2 t32 + 1 of every dimension tile
  const int64_t vbase = (int64_t)n_seq * S * (nq + nkv) * D + (int64_t)(seq * nkv + kv) * (D / 32) * (S / 16) * 512;
  for (int c = threadIdx.x; c < (D / 32) * 2 * 64; c += 256) {
    const int dt = c / 128, ksl = (c / 64) & 1, l = c & 63;
    const int j = 32 * dt + (l & 31), k0 = 16 * ksl + 8 * (l >> 5);
    u32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[e] = (uint32_t)t[j][k0 + 2 * e] | ((uint32_t)t[j][k0 + 2 * e + 1] << 16);
    *reinterpret_cast<u32x4*>(frag + vbase + ((int64_t)dt * (S / 16) + 2 * t32 + ksl) * 512 + l * 8) = x;
  }
}

static bool a16(const void* q) { return ((uintptr_t)q & 15) == 0; }

bool attn_fwd_ok(int S, int d, int64_t ld, int64_t ldo, const void* qkv, const void* O,
                 const void* frag) {
  return (d == 64 || d == 128) && S % QT == 0 && S >= QT && S <= SMAX && ld % 8 == 0 &&
         ldo % 4 == 0 && a16(qkv) && ((uintptr_t)O & 7) == 0 && a16(frag);
}

bool attn_bwd_ok(int S, int d, int64_t ld, int64_t lddo, int64_t ldq, const void* qkv,
                 const void* dO, const void* dQ, const void* frag, const void* Pin) {
  return (d == 64 || d == 128) && S % QT == 0 && S >= QT && S <= SMAX && ld % 8 == 0 &&
         lddo % 8 == 0 && ldq % 4 == 0 && a16(qkv) && a16(dO) && a16(dQ) && a16(frag) && a16(Pin);
}

template <bool BWD>
static hipError_t attn_launch(const AttnK& k, const PrepSrc& s0, const PrepSrc& s1,
                              const PrepSrc& s2, int d, hipStream_t s) {
  const dim3 pgrid(k.S / 32, k.n_seq, k.nq + 2 * k.nkv), grid(k.S / QT, k.n_seq * k.nq);
  uint16_t* frag = const_cast<uint16_t*>(k.frag);
  if (d == 128) {
    hipLaunchKernelGGL(attn_prep_k<128>, pgrid, dim3(256), 0, s, s0, s1, s2, k.S, k.n_seq, k.nq,
                       k.nkv, frag);
    hipLaunchKernelGGL((attn_k<128, BWD>), grid, dim3(64 * NW), 0, s, k);
  } else {
    hipLaunchKernelGGL(attn_prep_k<64>, pgrid, dim3(256), 0, s, s0, s1, s2, k.S, k.n_seq, k.nq,
                       k.nkv, frag);
    hipLaunchKernelGGL((attn_k<64, BWD>), grid, dim3(64 * NW), 0, s, k);
  }
  return hipGetLastError();
}

hipError_t attn_fwd(const AttnFwdParams& p, int d, hipStream_t s) {
  AttnK k{};
  k.frag = p.frag; k.Pf = p.Pf; k.Pb = p.Pb; k.O = p.O; k.ldo = p.ldo;
  k.n_seq = p.n_seq; k.S = p.S; k.nq = p.nq; k.nkv = p.nkv; k.alpha = p.alpha;
  // regions: q, k, v^T
  const PrepSrc s0{p.qkv, p.ld, 0}, s1{p.qkv, p.ld, (int64_t)p.nq * d},
      s2{p.qkv, p.ld, (int64_t)(p.nq + p.nkv) * d};
  return attn_launch<false>(k, s0, s1, s2, d, s);
}

hipError_t attn_bwd(const AttnBwdParams& p, int d, hipStream_t s) {
  AttnK k{};
  k.frag = p.frag; k.Pin = p.Pin; k.Pb = p.dS; k.dQ = p.dQ; k.ldq = p.ldq;
  k.n_seq = p.n_seq; k.S = p.S; k.nq = p.nq; k.nkv = p.nkv; k.alpha = p.alpha;
  // regions: dO, v, k^T
  const PrepSrc s0{p.dO, p.lddo, 0}, s1{p.qkv, p.ld, (int64_t)(p.nq + p.nkv) * d},
      s2{p.qkv, p.ld, (int64_t)p.nq * d};
  return attn_launch<true>(k, s0, s1, s2, d, s);
}

}  // namespace lsn
