// Causal grouped-query attention forward in one kernel per layer pass:
//
//   S = alpha q k^T (keys <= query), P = softmax(S) over the row, O = P v
//
// One workgroup (four waves) per (sequence, q head, 64-query tile).  The
// tile's scores for its keys 0 .. q0 + 63 live in LDS (fp32, at most 64 x 512:
// 129 KiB), so the scores never round-trip through HBM; only O (bf16) and,
// in the backward's recompute, the probabilities the backward reads (P in
// fp32 for the softmax gradient, P in bf16 for dV) are written.
//
// Phase 1 (scores): MFMA v_mfma_f32_32x32x16_bf16 with the keys as the first
// operand and the queries as the second, so a lane's accumulators are four
// consecutive keys of one query row: one 16-byte LDS store each.  Wave w
// takes the 32-key tiles j = w, w + 4, ... of the tile's causal extent.
// Phase 2 (softmax): wave w owns rows 16 w .. 16 w + 15; per row the same
// arithmetic as the two-pass softmax kernel (max and sum over keys <= query,
// one exp per element); P (bf16) overwrites the front half of the row.
// Phase 3 (O^T = v^T P^T): the first operand is v^T, read from a transposed
// copy vT [seq][kv head][d][S] (an MFMA operand needs 8 consecutive keys per
// lane), the second is P from LDS; a lane's accumulators are four
// consecutive head dimensions of one query: one 8-byte bf16 store each.
//
// Every output is written by one lane after a fixed-order reduction:
// results are deterministic and the same with or without the P outputs.
#include "common.h"

#include "attn.h"

namespace lsn {

namespace {
constexpr int QT = 64;          // queries per workgroup
constexpr int SMAX = 512;       // longest sequence the LDS score tile holds
constexpr int RS = SMAX + 4;    // LDS row stride (floats): rows 4 banks apart
}  // namespace

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_k(const AttnFwdParams p) {
  constexpr int KS = D / 16;  // MFMA k-steps over the head dimension
  __shared__ __attribute__((aligned(16))) float sS[QT * RS];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  const int S = p.S, nq = p.nq;
  const int qt = blockIdx.x, z = blockIdx.y;
  const int seq = z / nq, h = z % nq, kvh = h / (nq / p.nkv);
  const int q0 = qt * QT, nk = q0 + QT;  // keys 0 .. nk - 1
  const int64_t ld = p.ld;
  const uint16_t* Q = p.qkv + ((int64_t)seq * S + q0) * ld + h * D;
  const uint16_t* Kp = p.qkv + (int64_t)seq * S * ld + (int64_t)nq * D + kvh * D;

  // ---- phase 1: scores of the tile's 64 queries against keys < nk ----
  {
    bf16x8 qf[2][KS];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        qf[i][kk] = *reinterpret_cast<const bf16x8*>(Q + (int64_t)(32 * i + lr) * ld + 16 * kk + 8 * hh);
    const int nkt = nk / 32;
    bf16x8 kf[SMAX / 128][KS];
#pragma unroll
    for (int jj = 0; jj < SMAX / 128; ++jj) {
      const int j = w + 4 * jj;
      if (j < nkt)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          kf[jj][kk] = *reinterpret_cast<const bf16x8*>(Kp + (int64_t)(32 * j + lr) * ld + 16 * kk + 8 * hh);
    }
#pragma unroll
    for (int jj = 0; jj < SMAX / 128; ++jj) {
      const int j = w + 4 * jj;
      if (j >= nkt) continue;
      f32x16 acc[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[jj][kk], qf[i][kk], acc[i], 0, 0, 0);
      // acc[i][4 g + t]: query 32 i + lr, key 32 j + 8 g + 4 hh + t
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = {p.alpha * acc[i][4 * g], p.alpha * acc[i][4 * g + 1],
                           p.alpha * acc[i][4 * g + 2], p.alpha * acc[i][4 * g + 3]};
          *reinterpret_cast<f32x4*>(&sS[(32 * i + lr) * RS + 32 * j + 8 * g + 4 * hh]) = v;
        }
    }
  }
  __syncthreads();

  // ---- phase 2: causal softmax of the 64 rows ----
  for (int rr = 0; rr < QT / 4; ++rr) {
    const int r = w * (QT / 4) + rr, i = q0 + r;  // i: query position in the sequence
    float* row = &sS[r * RS];
    f32x4 v[SMAX / 256];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < SMAX / 256; ++u) {
      const int c = lane + 64 * u;
      v[u] = 4 * c < nk ? *reinterpret_cast<const f32x4*>(row + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * c + e <= i) m = fmaxf(m, v[u][e]);
    }
    m = wave_max(m);
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < SMAX / 256; ++u) {
      const int c = lane + 64 * u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ex = 4 * c + e <= i ? expf(v[u][e] - m) : 0.f;
        v[u][e] = ex;
        sum += ex;
      }
    }
    sum = wave_sum(sum);
    const float inv = 1.0f / sum;
    const int64_t prow = ((int64_t)z * S + i) * S;  // row i of head z in Pf / Pb
#pragma unroll
    for (int u = 0; u < SMAX / 256; ++u) {
      const int c = lane + 64 * u;
      if (4 * c >= nk) continue;
      const f32x4 pv = v[u] * inv;
      const u32x2 pb = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
      // bf16 P over the front half of the row: every lane's reads of this
      // row precede (through m and sum) every write
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(row) + 4 * c) = pb;
      if (p.Pf) *reinterpret_cast<f32x4*>(p.Pf + prow + 4 * c) = pv;
      if (p.Pb) *reinterpret_cast<u32x2*>(p.Pb + prow + 4 * c) = pb;
    }
    if (p.Pb)  // keys beyond the tile's extent: zero
      for (int c = nk / 4 + lane; c < S / 4; c += 64)
        *reinterpret_cast<u32x2*>(p.Pb + prow + 4 * c) = u32x2{0u, 0u};
  }
  __syncthreads();

  // ---- phase 3: O^T[d][q] = sum over keys of v^T[d][key] P^T[key][q] ----
  {
    constexpr int NDT = D / 32;            // 32-wide head-dimension tiles
    constexpr int QPW = NDT == 4 ? 2 : 1;  // query tiles per wave
    const int dt = w % NDT, qi0 = NDT == 4 ? 0 : w / NDT;
    const uint16_t* vT = p.vT + (((int64_t)seq * p.nkv + kvh) * D + dt * 32 + lr) * S + 8 * hh;
    const int nks = nk / 16;
    bf16x8 vf[SMAX / 16];
#pragma unroll
    for (int ks = 0; ks < SMAX / 16; ++ks)
      if (ks < nks) vf[ks] = *reinterpret_cast<const bf16x8*>(vT + 16 * ks);
    f32x16 acc[QPW];
#pragma unroll
    for (int a = 0; a < QPW; ++a)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][e] = 0.f;
    const char* sP = reinterpret_cast<const char*>(sS);
#pragma unroll
    for (int ks = 0; ks < SMAX / 16; ++ks) {
#pragma unroll
      for (int a = 0; a < QPW; ++a) {
        const int qi = qi0 + a;
        // query tile qi sees keys <= q0 + 32 qi + 31 only (P is zero beyond)
        if (ks >= nks || 16 * ks >= q0 + 32 * qi + 32) continue;
        const bf16x8 pf = *reinterpret_cast<const bf16x8*>(
            sP + (size_t)(32 * qi + lr) * RS * 4 + (16 * ks + 8 * hh) * 2);
        acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks], pf, acc[a], 0, 0, 0);
      }
    }
    // acc[a][4 g + t]: head dimension dt 32 + 8 g + 4 hh + t, query 32 qi + lr
#pragma unroll
    for (int a = 0; a < QPW; ++a) {
      uint16_t* o = p.O + ((int64_t)seq * S + q0 + 32 * (qi0 + a) + lr) * p.ldo + h * D + dt * 32 + 4 * hh;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<u32x2*>(o + 8 * g) =
            u32x2{pack_bf16x2(acc[a][4 * g], acc[a][4 * g + 1]),
                  pack_bf16x2(acc[a][4 * g + 2], acc[a][4 * g + 3])};
    }
  }
}

// vT[seq][kv][j][s] = v[seq S + s][kv d + j]: one 64-token x d tile per block
// through LDS (16-byte global loads and stores)
template <int D>
__global__ __launch_bounds__(256) void vtrans_k(const uint16_t* __restrict__ qkv, int64_t ld,
                                                int64_t voff, int S, int nkv,
                                                uint16_t* __restrict__ vT) {
  __shared__ uint16_t t[D][64 + 8];
  const int s0 = blockIdx.x * 64, sk = blockIdx.y;  // sk = seq nkv + kv
  const int seq = sk / nkv, kv = sk % nkv;
  const uint16_t* src = qkv + ((int64_t)seq * S + s0) * ld + voff + (int64_t)kv * D;
  for (int c = threadIdx.x; c < 64 * D / 8; c += 256) {
    const int tok = c / (D / 8), j0 = (c % (D / 8)) * 8;
    const u32x4 x = *reinterpret_cast<const u32x4*>(src + (int64_t)tok * ld + j0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t[j0 + 2 * e][tok] = (uint16_t)(x[e] & 0xFFFFu);
      t[j0 + 2 * e + 1][tok] = (uint16_t)(x[e] >> 16);
    }
  }
  __syncthreads();
  uint16_t* dst = vT + ((int64_t)sk * D) * S + s0;
  for (int c = threadIdx.x; c < D * 8; c += 256) {
    const int j = c / 8, k0 = (c % 8) * 8;
    u32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[e] = (uint32_t)t[j][k0 + 2 * e] | ((uint32_t)t[j][k0 + 2 * e + 1] << 16);
    *reinterpret_cast<u32x4*>(dst + (int64_t)j * S + k0) = x;
  }
}

static bool a16(const void* q) { return ((uintptr_t)q & 15) == 0; }

bool attn_fwd_ok(int S, int d, int64_t ld, int64_t ldo, const void* qkv, const void* O,
                 const void* vT) {
  return (d == 64 || d == 128) && S % QT == 0 && S >= QT && S <= SMAX && ld % 8 == 0 &&
         ldo % 4 == 0 && a16(qkv) && ((uintptr_t)O & 7) == 0 && a16(vT);
}

hipError_t attn_fwd(const AttnFwdParams& p, int n_seq, int d, hipStream_t s) {
  const dim3 tgrid(p.S / 64, n_seq * p.nkv), grid(p.S / QT, n_seq * p.nq);
  const int64_t voff = (int64_t)(p.nq + p.nkv) * d;
  if (d == 128) {
    hipLaunchKernelGGL(vtrans_k<128>, tgrid, dim3(256), 0, s, p.qkv, p.ld, voff, p.S, p.nkv,
                       const_cast<uint16_t*>(p.vT));
    hipLaunchKernelGGL(attn_fwd_k<128>, grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL(vtrans_k<64>, tgrid, dim3(256), 0, s, p.qkv, p.ld, voff, p.S, p.nkv,
                       const_cast<uint16_t*>(p.vT));
    hipLaunchKernelGGL(attn_fwd_k<64>, grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace lsn
