// Per-layer kernels around the GEMMs: RMSNorm, RoPE, causal softmax, SwiGLU,
// embedding gather, LoRA operand packing, the vocabulary-chunk log-softmax,
// losses, SGD, NF4 dequantization and small converters.
//
// Every reduction runs in a fixed order (one owner thread, or a fixed
// butterfly + fixed cross-wave order), with no atomics, so a run is
// bit-reproducible and independent of where the weights live.
#include "common.h"
#include "ops.h"

#include <type_traits>

namespace lsn {

// ---------------------------------------------------------------------------
// RMSNorm: y = g * h / sqrt(mean(h^2) + eps); one block per row
// ---------------------------------------------------------------------------
__global__ void rmsnorm_fwd_k(const float* __restrict__ h, const uint16_t* __restrict__ g, int H,
                              float eps, uint16_t* __restrict__ y, float* __restrict__ rstd) {
  __shared__ float red[16];
  const int64_t row = blockIdx.x;
  const float* x = h + row * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += blockDim.x) ss += x[i] * x[i];
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  if (threadIdx.x == 0) rstd[row] = r;
  for (int i = threadIdx.x; i < H; i += blockDim.x)
    y[row * H + i] = f32_to_bf16_bits(bf16_to_f32(g[i]) * (x[i] * r));
}

// out = dres + rstd*(g dy) - rstd^3/H * h * sum(g dy h)
__global__ void rmsnorm_bwd_k(const float* __restrict__ h, const uint16_t* __restrict__ g,
                              const float* __restrict__ rstd, const float* __restrict__ dy,
                              const float* dres, int H, float* out) {
  __shared__ float red[16];
  const int64_t row = blockIdx.x;
  const float* x = h + row * H;
  const float* d = dy + row * H;
  float dot = 0.f;
  for (int i = threadIdx.x; i < H; i += blockDim.x) dot += bf16_to_f32(g[i]) * d[i] * x[i];
  dot = block_sum(dot, red);
  const float r = rstd[row];
  const float c = r * r * r * dot / (float)H;
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    const float v = r * bf16_to_f32(g[i]) * d[i] - c * x[i];
    out[row * H + i] = (dres ? dres[row * H + i] : 0.f) + v;
  }
}

// ---------------------------------------------------------------------------
// RoPE (rotate-half) on the fused q|k|v rows.  Position = token % S.
// fwd: fp32 q,k,v -> bf16 rotated q, k and plain v.
// bwd: fp32 dq,dk,dv rotated back in place (fp32) + bf16 copy of all three.
// ---------------------------------------------------------------------------
LSN_DEV void rope_angle(int pos, int j, int d, float theta, float* c, float* s) {
  const float inv = powf(theta, -2.0f * (float)j / (float)d);
  sincosf((float)pos * inv, s, c);
}

__global__ void rope_fwd_k(const float* __restrict__ qkv, uint16_t* __restrict__ out, int S,
                           int nq, int nkv, int d, float theta) {
  const int64_t t = blockIdx.x;
  const int pos = (int)(t % S);
  const int W = (nq + 2 * nkv) * d;
  const int half = d / 2;
  const float* x = qkv + t * W;
  uint16_t* y = out + t * W;
  const int nrot = (nq + nkv) * half;  // rotated pairs
  for (int i = threadIdx.x; i < nrot; i += blockDim.x) {
    const int head = i / half, j = i % half;
    float c, s;
    rope_angle(pos, j, d, theta, &c, &s);
    const float x1 = x[head * d + j], x2 = x[head * d + j + half];
    y[head * d + j] = f32_to_bf16_bits(x1 * c - x2 * s);
    y[head * d + j + half] = f32_to_bf16_bits(x2 * c + x1 * s);
  }
  for (int i = threadIdx.x; i < nkv * d; i += blockDim.x) {
    const int o = (nq + nkv) * d + i;
    y[o] = f32_to_bf16_bits(x[o]);
  }
}

__global__ void rope_bwd_k(float* __restrict__ dqkv, uint16_t* __restrict__ outb, int S, int nq,
                           int nkv, int d, float theta) {
  const int64_t t = blockIdx.x;
  const int pos = (int)(t % S);
  const int W = (nq + 2 * nkv) * d;
  const int half = d / 2;
  float* x = dqkv + t * W;
  uint16_t* y = outb + t * W;
  const int nrot = (nq + nkv) * half;
  for (int i = threadIdx.x; i < nrot; i += blockDim.x) {
    const int head = i / half, j = i % half;
    float c, s;
    rope_angle(pos, j, d, theta, &c, &s);
    const float d1 = x[head * d + j], d2 = x[head * d + j + half];
    const float r1 = d1 * c + d2 * s, r2 = d2 * c - d1 * s;
    x[head * d + j] = r1;
    x[head * d + j + half] = r2;
    y[head * d + j] = f32_to_bf16_bits(r1);
    y[head * d + j + half] = f32_to_bf16_bits(r2);
  }
  for (int i = threadIdx.x; i < nkv * d; i += blockDim.x) {
    const int o = (nq + nkv) * d + i;
    y[o] = f32_to_bf16_bits(x[o]);
  }
}

// ---------------------------------------------------------------------------
// causal softmax over rows of [Z, S, S] scores (already scaled); one wave
// per row.  Writes P in fp32 and bf16, zeros above the diagonal.
// ---------------------------------------------------------------------------
__global__ void softmax_causal_k(const float* __restrict__ sc, float* __restrict__ Pf,
                                 uint16_t* __restrict__ Pb, int S, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int i = (int)(row % S);
  const float* x = sc + row * S;
  float m = -INFINITY;
  for (int j = lane; j <= i; j += 64) m = fmaxf(m, x[j]);
  m = wave_max(m);
  float sum = 0.f;
  for (int j = lane; j <= i; j += 64) sum += expf(x[j] - m);
  sum = wave_sum(sum);
  const float inv = 1.0f / sum;
  for (int j = lane; j < S; j += 64) {
    const float p = (j <= i) ? expf(x[j] - m) * inv : 0.f;
    Pf[row * S + j] = p;
    Pb[row * S + j] = f32_to_bf16_bits(p);
  }
}

// dS = P * (dP - sum_j dP*P) -> bf16; one wave per row
__global__ void softmax_bwd_k(const float* __restrict__ Pf, const float* __restrict__ dP,
                              uint16_t* __restrict__ dS, int S, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int i = (int)(row % S);
  const float* p = Pf + row * S;
  const float* g = dP + row * S;
  float dot = 0.f;
  for (int j = lane; j <= i; j += 64) dot += p[j] * g[j];
  dot = wave_sum(dot);
  for (int j = lane; j < S; j += 64)
    dS[row * S + j] = f32_to_bf16_bits((j <= i) ? p[j] * (g[j] - dot) : 0.f);
}

// ---------------------------------------------------------------------------
// SwiGLU on the fused gate|up rows [T, 2F]
// ---------------------------------------------------------------------------
LSN_DEV float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }

__global__ void swiglu_fwd_k(const float* __restrict__ gu, uint16_t* __restrict__ a, int F,
                             int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t t = i / F, f = i % F;
  const float g = gu[t * 2 * F + f], u = gu[t * 2 * F + F + f];
  a[i] = f32_to_bf16_bits(swiglu_act(g, u));
}

// dg = da * u * silu'(g), du = da * silu(g) -> bf16 [T, 2F] (+ fp32 copy)
__global__ void swiglu_bwd_k(const float* __restrict__ gu, const float* __restrict__ da,
                             uint16_t* __restrict__ dgu, float* __restrict__ dguf, int F,
                             int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t t = i / F, f = i % F;
  const float g = gu[t * 2 * F + f], u = gu[t * 2 * F + F + f];
  const float s = sigm(g);
  const float dg = da[i] * u * (s * (1.0f + g * (1.0f - s)));
  const float du = da[i] * (g * s);
  dgu[t * 2 * F + f] = f32_to_bf16_bits(dg);
  dgu[t * 2 * F + F + f] = f32_to_bf16_bits(du);
  if (dguf) {
    dguf[t * 2 * F + f] = dg;
    dguf[t * 2 * F + F + f] = du;
  }
}

// ---------------------------------------------------------------------------
// embedding rows (bf16 table) -> fp32
// ---------------------------------------------------------------------------
// a token id outside [0, V) yields a NaN row instead of an out-of-bounds read
__global__ void embed_k(const int32_t* __restrict__ tok, const uint16_t* __restrict__ table,
                        int H, int V, float* __restrict__ h) {
  const int64_t t = blockIdx.x;
  const int64_t v = tok[t];
  const bool ok = v >= 0 && v < V;
  for (int i = threadIdx.x; i < H; i += blockDim.x)
    h[t * H + i] = ok ? bf16_to_f32(table[v * H + i]) : __builtin_nanf("");
}


// ---------------------------------------------------------------------------
// vocabulary-chunk log-softmax (online max / sum) and target gather
// ---------------------------------------------------------------------------
// lse = m + log(sum); logp at the target; inv (when given) = 1 / sum.  A
// negative target means "no target" (logp 0); a target >= V is not a
// vocabulary entry and yields NaN, which the losses propagate.
__global__ void lse_final_k(const float* __restrict__ run_m, const float* __restrict__ run_s,
                            const float* __restrict__ tlogit, const int32_t* __restrict__ tgt,
                            int T, int V, float* __restrict__ logp, float* __restrict__ lse,
                            float* __restrict__ inv) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const float l = run_m[t] + logf(run_s[t]);
  lse[t] = l;
  const int y = tgt[t];
  logp[t] = y < 0 ? 0.f : y < V ? tlogit[t] - l : __builtin_nanf("");
  if (inv) inv[t] = 1.0f / run_s[t];
}

// Chunk pass of the LM head.  With m the running max before the chunk, M
// the chunk max and m' = max(m, M): the chunk's sum of exp(l - m') is merged
// into the running sum as sum * alpha + chunk sum with alpha = exp(m - m').
// One block of 256 threads per row; the row is read twice (max, then the
// exponentials), each thread in a fixed order, then fixed-order block sums.
// ACC (the pass that keeps the backward's state) also writes alpha, which
// rescales the expected-row accumulator, and p~ = bf16(exp(l - m')) [T, Vc]
// for the accumulator GEMM; the sums are the same bits either way.
template <bool ACC>
__global__ void lse_chunk_k(const float* __restrict__ logits, int Vc, int v0,
                            const int32_t* __restrict__ tgt, float* __restrict__ run_m,
                            float* __restrict__ run_s, float* __restrict__ tlogit,
                            float* __restrict__ alpha, uint16_t* __restrict__ pt, int first) {
  __shared__ float red[16];
  const int64_t t = blockIdx.x;
  const float* x = logits + t * Vc;
  uint16_t* o = ACC ? pt + t * Vc : nullptr;
  const bool vec = Vc % 8 == 0;  // 16-byte rows of logits and of p~
  float mx = -INFINITY;
  if (vec) {
    const f32x4* x4 = reinterpret_cast<const f32x4*>(x);
    for (int i = threadIdx.x; i < Vc / 4; i += blockDim.x) {
      const f32x4 v = x4[i];
      mx = fmaxf(mx, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    }
  } else {
    for (int i = threadIdx.x; i < Vc; i += blockDim.x) mx = fmaxf(mx, x[i]);
  }
  const float M = block_max(mx, red);
  const float mo = first ? -INFINITY : run_m[t];
  const float mn = fmaxf(mo, M);
  float sum = 0.f;
  if (vec) {
    const f32x4* x4 = reinterpret_cast<const f32x4*>(x);
    for (int i = threadIdx.x; i < Vc / 8; i += blockDim.x) {
      const f32x4 a = x4[2 * i], b2 = x4[2 * i + 1];
      float e[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        e[q] = expf((q < 4 ? a[q] : b2[q - 4]) - mn);
        sum += e[q];
      }
      if constexpr (ACC) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(e[2 * q], e[2 * q + 1]);
        reinterpret_cast<u32x4*>(o)[i] = w;
      }
    }
  } else {
    for (int i = threadIdx.x; i < Vc; i += blockDim.x) {
      const float e = expf(x[i] - mn);
      sum += e;
      if constexpr (ACC) o[i] = f32_to_bf16_bits(e);
    }
  }
  const float S = block_sum(sum, red);
  if (threadIdx.x == 0) {
    const float al = first ? 0.f : expf(mo - mn);
    run_s[t] = first ? S : run_s[t] * al + S;
    run_m[t] = mn;
    if constexpr (ACC) alpha[t] = al;
    if (first) tlogit[t] = 0.f;
    const int y = tgt[t];
    if (y >= v0 && y < v0 + Vc) tlogit[t] = x[y - v0];
  }
}

// x[t, :] *= f[t] over rows of n columns (n % 4 == 0, 16-byte aligned rows)
__global__ void scale_rows_k(f32x4* __restrict__ x, const float* __restrict__ f, int n4,
                             int64_t total4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total4) return;
  x[i] = x[i] * f[i / n4];
}

__global__ void scale_rows1_k(float* __restrict__ x, const float* __restrict__ f, int n,
                              int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < total) x[i] *= f[i / n];
}

// LM-head input gradient from the expected embedding row E (in place):
// dn[t, :] = dlogp[t] * (W[y_t, :] - E[t, :]); a position without a target
// has dlogp 0 and gets 0.  A target outside [0, V) reads no row of W (its
// log-prob is already NaN).
__global__ void head_grad_k(const float* __restrict__ dlogp, const int32_t* __restrict__ tgt,
                            const uint16_t* __restrict__ W, int H, int V, int64_t n,
                            float* __restrict__ E) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t t = i / H;
  const int y = tgt[t];
  const float wy = (y >= 0 && y < V) ? bf16_to_f32(W[(int64_t)y * H + (i - t * H)]) : 0.f;
  E[i] = dlogp[t] * (wy - E[i]);
}

// ---------------------------------------------------------------------------
// losses (single block, fixed-order reductions)
// ---------------------------------------------------------------------------
__global__ void sft_loss_k(const float* __restrict__ logp, const int32_t* __restrict__ tgt, int n,
                           float* __restrict__ loss, float* __restrict__ dlogp) {
  __shared__ float red[16];
  float s = 0.f, c = 0.f;
  for (int i = threadIdx.x; i < n; i += blockDim.x)
    if (tgt[i] >= 0) {
      s += logp[i];
      c += 1.f;
    }
  s = block_sum(s, red);
  c = block_sum(c, red);
  if (threadIdx.x == 0) loss[0] = -s / c;
  const float g = -1.0f / c;
  for (int i = threadIdx.x; i < n; i += blockDim.x) dlogp[i] = (tgt[i] >= 0) ? g : 0.f;
}

// Preference losses on one pair laid out as two sequences (chosen, rejected)
// of S tokens; response targets at positions P-1 .. S-2 (n = S-P each).
// kind 0 DPO:   z = beta((pc-rc)-(pr-rr)),  loss = softplus(-z)
// kind 1 SimPO: u = beta(pc/n - pr/n) - p2, loss = softplus(-u)
// kind 2 ORPO:  v = lo(pc/n) - lo(pr/n), lo(m) = m - log(1-e^m),
//               loss = -pc/n + p2 softplus(-v)
// kind 3 KTO:   loss = (1 - sig(beta(pc-rc))) + (1 - sig(-beta(pr-rr)))
// out = {loss, z|u|v|pc-rc, pc, pr, rc, rr}; dlogp on response positions.
LSN_DEV float softplus_f(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }
LSN_DEV float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }

__global__ void pref_loss_k(int kind, const float* __restrict__ lp, const float* __restrict__ lr,
                            int S, int P, float beta, float p2, float* __restrict__ out,
                            float* __restrict__ dlogp) {
  __shared__ float red[16];
  float v[4] = {0.f, 0.f, 0.f, 0.f};  // pc, pr, rc, rr
  for (int i = threadIdx.x; i < 2 * S; i += blockDim.x) {
    const int seq = i / S, pos = i % S;
    if (pos >= P - 1 && pos <= S - 2) {
      v[seq] += lp[i];
      if (lr) v[2 + seq] += lr[i];
    }
  }
  for (int q = 0; q < 4; ++q) v[q] = block_sum(v[q], red);
  const float pc = v[0], pr = v[1], rc = v[2], rr = v[3];
  const float n = (float)(S - P);
  float loss = 0.f, aux = 0.f, gc = 0.f, gr = 0.f;
  if (kind == 0) {
    aux = beta * ((pc - rc) - (pr - rr));
    loss = softplus_f(-aux);
    const float g = beta * sigmoid_f(-aux);
    gc = -g;
    gr = g;
  } else if (kind == 1) {
    aux = beta * (pc / n - pr / n) - p2;
    loss = softplus_f(-aux);
    const float g = sigmoid_f(-aux) * beta / n;
    gc = -g;
    gr = g;
  } else if (kind == 2) {
    const float mc = pc / n, mr = pr / n;
    const float oc = -expm1f(mc), orr = -expm1f(mr);  // 1 - e^m
    aux = (mc - logf(oc)) - (mr - logf(orr));
    loss = -mc + p2 * softplus_f(-aux);
    const float g = p2 * sigmoid_f(-aux);
    gc = (-1.0f - g / oc) / n;
    gr = (g / orr) / n;
  } else {
    aux = pc - rc;
    const float sc = sigmoid_f(beta * aux), sr = sigmoid_f(-beta * (pr - rr));
    loss = (1.0f - sc) + (1.0f - sr);
    gc = -beta * sc * (1.0f - sc);
    gr = beta * sr * (1.0f - sr);
  }
  if (threadIdx.x == 0) {
    out[0] = loss;
    out[1] = aux;
    out[2] = pc;
    out[3] = pr;
    out[4] = rc;
    out[5] = rr;
  }
  for (int i = threadIdx.x; i < 2 * S; i += blockDim.x) {
    const int seq = i / S, pos = i % S;
    dlogp[i] = (pos >= P - 1 && pos <= S - 2) ? (seq == 0 ? gc : gr) : 0.f;
  }
}

// ---------------------------------------------------------------------------
// small utilities
// ---------------------------------------------------------------------------
__global__ void sgd_k(float* __restrict__ p, const float* __restrict__ g, float lr, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] -= lr * g[i];
}

// Grouped-query sum: out[(q * S + i) * ldo + kv * d + j] = sum over the grp
// q heads h of kv, in head order, of part[((q * nq + h) * S + i) * d + j]
// (q: sequence, i: position, j: feature; four features per thread).
__global__ void group_sum4_k(const f32x4* __restrict__ part, int nq, int grp, int S, int d4,
                             float* __restrict__ out, int64_t ldo, int64_t total4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total4) return;
  const int nkv = nq / grp;
  const int j4 = (int)(i % d4);
  int64_t r = i / d4;
  const int pos = (int)(r % S);
  r /= S;
  const int kv = (int)(r % nkv);
  const int64_t q = r / nkv;
  const f32x4* src = part + ((q * nq + (int64_t)kv * grp) * S + pos) * d4 + j4;
  f32x4 acc = src[0];
  for (int g = 1; g < grp; ++g) acc += src[(int64_t)g * S * d4];
  *reinterpret_cast<f32x4*>(out + (q * S + pos) * ldo + ((int64_t)kv * d4 + j4) * 4) = acc;
}

// One lane waits `ticks` periods of the device's constant-rate wall clock,
// then exits (a delay of bounded length on the stream it runs on).
__global__ void spin_k(uint64_t ticks) {
  if (threadIdx.x != 0) return;
  const uint64_t t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

__global__ void fill_k(uint32_t* __restrict__ p, uint32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void f32_to_bf16_k(const float* __restrict__ x, uint16_t* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = f32_to_bf16_bits(x[i]);
}
// four elements per thread (x 16-byte and y 8-byte aligned, n % 4 == 0)
__global__ void f32_to_bf16_x4_k(const f32x4* __restrict__ x, u32x2* __restrict__ y, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) {
    const f32x4 v = x[i];
    y[i] = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

// NF4 -> fp32 (bit-equal to the host codec) or bf16; 8 elements per thread
struct Levels {
  float v[16];
};
__global__ void nf4_dequant_k(const uint32_t* __restrict__ codes, const float* __restrict__ absmax,
                              int64_t nwords, Levels lv, float* __restrict__ of32,
                              u32x4* __restrict__ obf) {
  __shared__ float sl[16];
  if (threadIdx.x < 16) sl[threadIdx.x] = lv.v[threadIdx.x];
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nwords) return;
  const uint32_t w = codes[i];
  const float a = absmax[i >> 3];
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = sl[(w >> (4 * j)) & 15u] * a;
  if (of32) {
    f32x4* o = reinterpret_cast<f32x4*>(of32 + i * 8);
    o[0] = f32x4{v[0], v[1], v[2], v[3]};
    o[1] = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    obf[i] = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7])};
  }
}

// ---------------------------------------------------------------------------
// 16-byte forms of the kernels above, for rows whose length is a multiple of
// 4 (8 for softmax) and 16-byte aligned; same per-element arithmetic, each
// thread in a fixed order.  The launchers fall back to the scalar kernels
// for other shapes.
// ---------------------------------------------------------------------------
LSN_DEV float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
LSN_DEV float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
LSN_DEV bool al16(const void* q) { return ((uintptr_t)q & 15) == 0; }

// four consecutive elements of a SplitSum operand: the buffers added in
// split order from zero, as the split-k reduction adds them (one buffer: the
// value itself)
// value itself).  NS is the buffer count fixed at compile time (the
// launchers instantiate 1..8), so the loads of all buffers are issued
// before the first add; NS = 0 takes the run-time count a.ns, whose loop
// waits for each load in turn.
template <int NS>
LSN_DEV f32x4 sum4(const SplitSum& a, int64_t off) {
  if constexpr (NS == 1) {
    return *reinterpret_cast<const f32x4*>(a.p + off);
  } else if constexpr (NS == 0) {
    if (a.ns == 1) return *reinterpret_cast<const f32x4*>(a.p + off);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int y = 0; y < a.ns; ++y) acc += *reinterpret_cast<const f32x4*>(a.p + y * a.stride + off);
    return acc;
  } else {
    f32x4 v[NS];
#pragma unroll
    for (int y = 0; y < NS; ++y) v[y] = *reinterpret_cast<const f32x4*>(a.p + y * a.stride + off);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int y = 0; y < NS; ++y) acc += v[y];
    return acc;
  }
}

__global__ __launch_bounds__(256) void rmsnorm_fwd4_k(const float* __restrict__ h,
                                                      const uint16_t* __restrict__ g, int H,
                                                      float eps, uint16_t* __restrict__ y,
                                                      float* __restrict__ rstd) {
  __shared__ float red[16];
  const int64_t row = blockIdx.x;
  const f32x4* x = reinterpret_cast<const f32x4*>(h + row * H);
  const int n4 = H >> 2;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n4; i += 256) {
    const f32x4 v = x[i];
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  if (threadIdx.x == 0) rstd[row] = r;
  const u32x2* gw = reinterpret_cast<const u32x2*>(g);
  u32x2* yo = reinterpret_cast<u32x2*>(y + row * H);
  for (int i = threadIdx.x; i < n4; i += 256) {
    const f32x4 v = x[i];
    const u32x2 w = gw[i];
    yo[i] = u32x2{pack_bf16x2(bf_lo(w[0]) * (v[0] * r), bf_hi(w[0]) * (v[1] * r)),
                  pack_bf16x2(bf_lo(w[1]) * (v[2] * r), bf_hi(w[1]) * (v[3] * r))};
  }
}

// h = res + src (the residual add of a projection whose split-k partial sums
// src holds), written out, then RMSNorm of h as rmsnorm_fwd4_k
template <int NS>
__global__ __launch_bounds__(256) void rmsnorm_fwd_res4_k(const float* __restrict__ res,
                                                          const SplitSum src,
                                                          const uint16_t* __restrict__ g, int H,
                                                          float eps, float* __restrict__ hout,
                                                          uint16_t* __restrict__ y,
                                                          float* __restrict__ rstd) {
  __shared__ float red[16];
  const int64_t row = blockIdx.x;
  const f32x4* rr = reinterpret_cast<const f32x4*>(res + row * H);
  f32x4* x = reinterpret_cast<f32x4*>(hout + row * H);
  const int n4 = H >> 2;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n4; i += 256) {
    const f32x4 v = rr[i] + sum4<NS>(src, row * H + 4 * i);
    x[i] = v;
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  if (threadIdx.x == 0) rstd[row] = r;
  const u32x2* gw = reinterpret_cast<const u32x2*>(g);
  u32x2* yo = reinterpret_cast<u32x2*>(y + row * H);
  for (int i = threadIdx.x; i < n4; i += 256) {  // this thread's own writes above
    const f32x4 v = x[i];
    const u32x2 w = gw[i];
    yo[i] = u32x2{pack_bf16x2(bf_lo(w[0]) * (v[0] * r), bf_hi(w[0]) * (v[1] * r)),
                  pack_bf16x2(bf_lo(w[1]) * (v[2] * r), bf_hi(w[1]) * (v[3] * r))};
  }
}

// (dy: the output gradient, or the split-k partial sums of the GEMM that
// produced it, summed once: up to 8 chunks per thread stay in registers
// between the two passes; outb, if given, also receives bf16(out))
constexpr int RB_CACHE = 8;
template <int NS>
__global__ __launch_bounds__(256) void rmsnorm_bwd4_k(const float* __restrict__ h,
                                                      const uint16_t* __restrict__ g,
                                                      const float* __restrict__ rstd,
                                                      const SplitSum dy, const float* dres, int H,
                                                      float* out, uint16_t* __restrict__ outb) {
  __shared__ float red[16];
  const int64_t row = blockIdx.x;
  const f32x4* x = reinterpret_cast<const f32x4*>(h + row * H);
  const u32x2* gw = reinterpret_cast<const u32x2*>(g);
  const int n4 = H >> 2;
  f32x4 dc[RB_CACHE];
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < RB_CACHE; ++k) {
    const int i = threadIdx.x + 256 * k;
    if (i < n4) {
      const f32x4 xv = x[i], dv = sum4<NS>(dy, row * H + 4 * i);
      dc[k] = dv;
      const u32x2 w = gw[i];
      dot += bf_lo(w[0]) * dv[0] * xv[0] + bf_hi(w[0]) * dv[1] * xv[1] +
             bf_lo(w[1]) * dv[2] * xv[2] + bf_hi(w[1]) * dv[3] * xv[3];
    }
  }
  for (int i = threadIdx.x + 256 * RB_CACHE; i < n4; i += 256) {
    const f32x4 xv = x[i], dv = sum4<NS>(dy, row * H + 4 * i);
    const u32x2 w = gw[i];
    dot += bf_lo(w[0]) * dv[0] * xv[0] + bf_hi(w[0]) * dv[1] * xv[1] +
           bf_lo(w[1]) * dv[2] * xv[2] + bf_hi(w[1]) * dv[3] * xv[3];
  }
  dot = block_sum(dot, red);
  const float r = rstd[row];
  const float c = r * r * r * dot / (float)H;
  f32x4* o = reinterpret_cast<f32x4*>(out + row * H);
  const f32x4* dr = dres ? reinterpret_cast<const f32x4*>(dres + row * H) : nullptr;
  u32x2* ob = outb ? reinterpret_cast<u32x2*>(outb + row * H) : nullptr;
  auto emit = [&](int i, const f32x4& dv) {
    const f32x4 xv = x[i];
    const u32x2 w = gw[i];
    f32x4 v = {r * bf_lo(w[0]) * dv[0] - c * xv[0], r * bf_hi(w[0]) * dv[1] - c * xv[1],
               r * bf_lo(w[1]) * dv[2] - c * xv[2], r * bf_hi(w[1]) * dv[3] - c * xv[3]};
    if (dr) v = dr[i] + v;
    o[i] = v;
    if (ob) ob[i] = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  };
#pragma unroll
  for (int k = 0; k < RB_CACHE; ++k) {
    const int i = threadIdx.x + 256 * k;
    if (i < n4) emit(i, dc[k]);
  }
  for (int i = threadIdx.x + 256 * RB_CACHE; i < n4; i += 256) emit(i, sum4<NS>(dy, row * H + 4 * i));
}

// RoPE with the token's d/2 angles computed once per block into LDS.
// Forward: reads q|k|v from src (the projection's output or its split-k
// partial sums); backward: rotates xin in place.
template <bool FWD, int NS>
__global__ __launch_bounds__(256) void rope4_k(const SplitSum src, float* __restrict__ xin,
                                               uint16_t* __restrict__ out, int S, int nq,
                                               int nkv, int d, float theta) {
  __shared__ float sc[128], ss[128];
  const int64_t t = blockIdx.x;
  const int pos = (int)(t % S);
  const int W = (nq + 2 * nkv) * d, half = d / 2, h4 = half / 4;
  for (int j = threadIdx.x; j < half; j += 256) rope_angle(pos, j, d, theta, &sc[j], &ss[j]);
  __syncthreads();
  float* x = FWD ? nullptr : xin + t * W;
  uint16_t* y = out + t * W;
  auto ld4 = [&](int o) {
    return FWD ? sum4<NS>(src, t * W + o) : *reinterpret_cast<const f32x4*>(x + o);
  };
  const int nrot = (nq + nkv) * h4;  // 4-wide groups of rotated pairs
  for (int i = threadIdx.x; i < nrot; i += 256) {
    const int head = i / h4, j = (i % h4) * 4;
    const f32x4 a = ld4(head * d + j), b = ld4(head * d + j + half);
    f32x4 r1, r2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c = sc[j + e], s = ss[j + e];
      if (FWD) {
        r1[e] = a[e] * c - b[e] * s;
        r2[e] = b[e] * c + a[e] * s;
      } else {
        r1[e] = a[e] * c + b[e] * s;
        r2[e] = b[e] * c - a[e] * s;
      }
    }
    if (!FWD) {
      *reinterpret_cast<f32x4*>(x + head * d + j) = r1;
      *reinterpret_cast<f32x4*>(x + head * d + j + half) = r2;
    }
    *reinterpret_cast<u32x2*>(y + head * d + j) =
        u32x2{pack_bf16x2(r1[0], r1[1]), pack_bf16x2(r1[2], r1[3])};
    *reinterpret_cast<u32x2*>(y + head * d + j + half) =
        u32x2{pack_bf16x2(r2[0], r2[1]), pack_bf16x2(r2[2], r2[3])};
  }
  const int o0 = (nq + nkv) * d;
  for (int i = threadIdx.x; i < nkv * d / 4; i += 256) {
    const f32x4 v = ld4(o0 + 4 * i);
    reinterpret_cast<u32x2*>(y + o0)[i] = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

// Causal softmax, one wave per row, the row held in registers (NCH 16-byte
// chunks per lane, S <= 256 NCH): one exp per element.
template <int NCH>
__global__ __launch_bounds__(256) void softmax_causal4_k(const float* __restrict__ sc,
                                                         float* __restrict__ Pf,
                                                         uint16_t* __restrict__ Pb, int S,
                                                         int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int i = (int)(row % S), n4 = S >> 2;
  const f32x4* x = reinterpret_cast<const f32x4*>(sc + row * S);
  f32x4 v[NCH];
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < NCH; ++q) {
    const int c = lane + 64 * q;
    v[q] = (c < n4 && 4 * c <= i) ? x[c] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c < n4 && 4 * c + e <= i) m = fmaxf(m, v[q][e]);
  }
  m = wave_max(m);
  float sum = 0.f;
#pragma unroll
  for (int q = 0; q < NCH; ++q) {
    const int c = lane + 64 * q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ex = (c < n4 && 4 * c + e <= i) ? expf(v[q][e] - m) : 0.f;
      v[q][e] = ex;
      sum += ex;
    }
  }
  sum = wave_sum(sum);
  const float inv = 1.0f / sum;
  f32x4* pf = reinterpret_cast<f32x4*>(Pf + row * S);
  u32x2* pb = reinterpret_cast<u32x2*>(Pb + row * S);
#pragma unroll
  for (int q = 0; q < NCH; ++q) {
    const int c = lane + 64 * q;
    if (c >= n4) continue;
    const f32x4 p = v[q] * inv;
    pf[c] = p;
    pb[c] = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
  }
}

// dS = P (dP - sum_j dP P), one wave per row, 16-byte chunks
__global__ __launch_bounds__(256) void softmax_bwd4_k(const float* __restrict__ Pf,
                                                      const float* __restrict__ dP,
                                                      uint16_t* __restrict__ dS, int S,
                                                      int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int i = (int)(row % S), n4 = S >> 2;
  const f32x4* p = reinterpret_cast<const f32x4*>(Pf + row * S);
  const f32x4* g = reinterpret_cast<const f32x4*>(dP + row * S);
  float dot = 0.f;
  for (int c = lane; c < n4 && 4 * c <= i; c += 64) {
    const f32x4 pv = p[c], gv = g[c];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * c + e <= i) dot += pv[e] * gv[e];
  }
  dot = wave_sum(dot);
  u32x2* o = reinterpret_cast<u32x2*>(dS + row * S);
  for (int c = lane; c < n4; c += 64) {
    if (4 * c > i) {
      o[c] = u32x2{0u, 0u};
      continue;
    }
    const f32x4 pv = p[c], gv = g[c];
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (4 * c + e <= i) ? pv[e] * (gv[e] - dot) : 0.f;
    o[c] = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
  }
}

// SwiGLU, 4 features per thread; blockIdx.y = token
__global__ __launch_bounds__(256) void swiglu_fwd4_k(const float* __restrict__ gu,
                                                     uint16_t* __restrict__ a, int F) {
  const int f = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (f >= F) return;
  const int64_t t = blockIdx.y;
  const f32x4 g = *reinterpret_cast<const f32x4*>(gu + t * 2 * F + f);
  const f32x4 u = *reinterpret_cast<const f32x4*>(gu + t * 2 * F + F + f);
  float r[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = swiglu_act(g[e], u[e]);
  *reinterpret_cast<u32x2*>(a + t * F + f) = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
}

// (da: the gradient of a, or the split-k partial sums of the GEMM that
// produced it)
template <int NS>
__global__ __launch_bounds__(256) void swiglu_bwd4_k(const float* __restrict__ gu,
                                                     const SplitSum da,
                                                     uint16_t* __restrict__ dgu,
                                                     float* __restrict__ dguf, int F) {
  const int f = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (f >= F) return;
  const int64_t t = blockIdx.y;
  const f32x4 g = *reinterpret_cast<const f32x4*>(gu + t * 2 * F + f);
  const f32x4 u = *reinterpret_cast<const f32x4*>(gu + t * 2 * F + F + f);
  const f32x4 d = sum4<NS>(da, t * F + f);
  f32x4 dg, du;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float s = sigm(g[e]);
    dg[e] = d[e] * u[e] * (s * (1.0f + g[e] * (1.0f - s)));
    du[e] = d[e] * (g[e] * s);
  }
  *reinterpret_cast<u32x2*>(dgu + t * 2 * F + f) =
      u32x2{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
  *reinterpret_cast<u32x2*>(dgu + t * 2 * F + F + f) =
      u32x2{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
  if (dguf) {
    *reinterpret_cast<f32x4*>(dguf + t * 2 * F + f) = dg;
    *reinterpret_cast<f32x4*>(dguf + t * 2 * F + F + f) = du;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline unsigned nb(int64_t n, int b) { return (unsigned)((n + b - 1) / b); }

static bool a16(const void* q) { return ((uintptr_t)q & 15) == 0; }

void rmsnorm_fwd(const float* h, const uint16_t* g, int T, int H, float eps, uint16_t* y,
                 float* rstd, hipStream_t s) {
  if (H % 4 == 0 && a16(h) && ((uintptr_t)g & 7) == 0 && ((uintptr_t)y & 7) == 0)
    hipLaunchKernelGGL(rmsnorm_fwd4_k, dim3(T), dim3(256), 0, s, h, g, H, eps, y, rstd);
  else
    hipLaunchKernelGGL(rmsnorm_fwd_k, dim3(T), dim3(256), 0, s, h, g, H, eps, y, rstd);
}
void rmsnorm_bwd(const float* h, const uint16_t* g, const float* rstd, const float* dy,
                 const float* dres, int T, int H, float* out, hipStream_t s) {
  rmsnorm_bwd(h, g, rstd, SplitSum{dy, 1, 0}, dres, T, H, out, nullptr, s);
}
static bool split_vec(const SplitSum& a) { return a16(a.p) && a.stride % 4 == 0; }
// calls f with std::integral_constant<int, NS>: the split count 1..8, or 0
// (a run-time count) for more
template <class F>
static void with_splits(int ns, F&& f) {
  switch (ns) {
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 3: f(std::integral_constant<int, 3>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 5: f(std::integral_constant<int, 5>{}); break;
    case 6: f(std::integral_constant<int, 6>{}); break;
    case 7: f(std::integral_constant<int, 7>{}); break;
    case 8: f(std::integral_constant<int, 8>{}); break;
    default: f(std::integral_constant<int, 0>{}); break;
  }
}
bool rmsnorm_bwd_fuses(int H, const float* h, const float* out, const float* dres,
                       const uint16_t* g) {
  return H % 4 == 0 && a16(h) && a16(out) && (!dres || a16(dres)) && ((uintptr_t)g & 7) == 0;
}
void rmsnorm_bwd(const float* h, const uint16_t* g, const float* rstd, const SplitSum& dy,
                 const float* dres, int T, int H, float* out, uint16_t* outb, hipStream_t s) {
  if (rmsnorm_bwd_fuses(H, h, out, dres, g) && split_vec(dy) && ((uintptr_t)outb & 7) == 0) {
    with_splits(dy.ns, [&](auto ns) {
      hipLaunchKernelGGL((rmsnorm_bwd4_k<decltype(ns)::value>), dim3(T), dim3(256), 0, s, h, g,
                         rstd, dy, dres, H, out, outb);
    });
  } else if (dy.ns == 1) {
    hipLaunchKernelGGL(rmsnorm_bwd_k, dim3(T), dim3(256), 0, s, h, g, rstd, dy.p, dres, H, out);
    if (outb) f32_to_bf16(out, outb, (int64_t)T * H, s);
  }
}
bool rmsnorm_fwd_res_fuses(int H, const float* res, const float* hout, const uint16_t* g,
                           const uint16_t* y) {
  return H % 4 == 0 && a16(res) && a16(hout) && ((uintptr_t)g & 7) == 0 &&
         ((uintptr_t)y & 7) == 0;
}
void rmsnorm_fwd_res(const float* res, const SplitSum& src, const uint16_t* g, int T, int H,
                     float eps, float* hout, uint16_t* y, float* rstd, hipStream_t s) {
  with_splits(src.ns, [&](auto ns) {
    hipLaunchKernelGGL((rmsnorm_fwd_res4_k<decltype(ns)::value>), dim3(T), dim3(256), 0, s, res,
                       src, g, H, eps, hout, y, rstd);
  });
}
static bool rope_vec(const void* x, const void* y, int d) {
  return d % 8 == 0 && d / 2 <= 128 && a16(x) && ((uintptr_t)y & 7) == 0;
}
bool rope_fwd_fuses(int d, const uint16_t* out) { return rope_vec(out, out, d); }
void rope_fwd(const float* qkv, uint16_t* out, int T, int S, int nq, int nkv, int d, float theta,
              hipStream_t s) {
  rope_fwd(SplitSum{qkv, 1, 0}, out, T, S, nq, nkv, d, theta, s);
}
void rope_fwd(const SplitSum& qkv, uint16_t* out, int T, int S, int nq, int nkv, int d,
              float theta, hipStream_t s) {
  if (rope_vec(qkv.p, out, d) && split_vec(qkv))
    with_splits(qkv.ns, [&](auto ns) {
      hipLaunchKernelGGL((rope4_k<true, decltype(ns)::value>), dim3(T), dim3(256), 0, s, qkv,
                         nullptr, out, S, nq, nkv, d, theta);
    });
  else if (qkv.ns == 1)
    hipLaunchKernelGGL(rope_fwd_k, dim3(T), dim3(256), 0, s, qkv.p, out, S, nq, nkv, d, theta);
}
void rope_bwd(float* dqkv, uint16_t* outb, int T, int S, int nq, int nkv, int d, float theta,
              hipStream_t s) {
  if (rope_vec(dqkv, outb, d))
    hipLaunchKernelGGL((rope4_k<false, 1>), dim3(T), dim3(256), 0, s, SplitSum{}, dqkv, outb, S,
                       nq, nkv, d, theta);
  else
    hipLaunchKernelGGL(rope_bwd_k, dim3(T), dim3(256), 0, s, dqkv, outb, S, nq, nkv, d, theta);
}
void softmax_causal(const float* sc, float* Pf, uint16_t* Pb, int S, int64_t rows,
                    hipStream_t s) {
  const bool vec = S % 8 == 0 && a16(sc) && a16(Pf) && ((uintptr_t)Pb & 7) == 0;
  const dim3 grid(nb(rows, 4)), blk(256);
  if (vec && S <= 256) hipLaunchKernelGGL(softmax_causal4_k<1>, grid, blk, 0, s, sc, Pf, Pb, S, rows);
  else if (vec && S <= 512) hipLaunchKernelGGL(softmax_causal4_k<2>, grid, blk, 0, s, sc, Pf, Pb, S, rows);
  else if (vec && S <= 1024) hipLaunchKernelGGL(softmax_causal4_k<4>, grid, blk, 0, s, sc, Pf, Pb, S, rows);
  else if (vec && S <= 2048) hipLaunchKernelGGL(softmax_causal4_k<8>, grid, blk, 0, s, sc, Pf, Pb, S, rows);
  else hipLaunchKernelGGL(softmax_causal_k, grid, blk, 0, s, sc, Pf, Pb, S, rows);
}
void softmax_bwd(const float* Pf, const float* dP, uint16_t* dS, int S, int64_t rows,
                 hipStream_t s) {
  if (S % 8 == 0 && a16(Pf) && a16(dP) && ((uintptr_t)dS & 7) == 0)
    hipLaunchKernelGGL(softmax_bwd4_k, dim3(nb(rows, 4)), dim3(256), 0, s, Pf, dP, dS, S, rows);
  else
    hipLaunchKernelGGL(softmax_bwd_k, dim3(nb(rows, 4)), dim3(256), 0, s, Pf, dP, dS, S, rows);
}
void swiglu_fwd(const float* gu, uint16_t* a, int T, int F, hipStream_t s) {
  if (F % 4 == 0 && T <= 65535 && a16(gu) && ((uintptr_t)a & 7) == 0) {
    hipLaunchKernelGGL(swiglu_fwd4_k, dim3(nb(F / 4, 256), T), dim3(256), 0, s, gu, a, F);
    return;
  }
  const int64_t n = (int64_t)T * F;
  hipLaunchKernelGGL(swiglu_fwd_k, dim3(nb(n, 256)), dim3(256), 0, s, gu, a, F, n);
}
bool swiglu_bwd_fuses(int T, int F, const float* gu, const uint16_t* dgu, const float* dguf) {
  return F % 4 == 0 && T <= 65535 && a16(gu) && ((uintptr_t)dgu & 7) == 0 && (!dguf || a16(dguf));
}
void swiglu_bwd(const float* gu, const float* da, uint16_t* dgu, float* dguf, int T, int F,
                hipStream_t s) {
  swiglu_bwd(gu, SplitSum{da, 1, 0}, dgu, dguf, T, F, s);
}
void swiglu_bwd(const float* gu, const SplitSum& da, uint16_t* dgu, float* dguf, int T, int F,
                hipStream_t s) {
  if (swiglu_bwd_fuses(T, F, gu, dgu, dguf) && split_vec(da)) {
    with_splits(da.ns, [&](auto ns) {
      hipLaunchKernelGGL((swiglu_bwd4_k<decltype(ns)::value>), dim3(nb(F / 4, 256), T), dim3(256),
                         0, s, gu, da, dgu, dguf, F);
    });
    return;
  }
  if (da.ns != 1) return;
  const int64_t n = (int64_t)T * F;
  hipLaunchKernelGGL(swiglu_bwd_k, dim3(nb(n, 256)), dim3(256), 0, s, gu, da.p, dgu, dguf, F, n);
}
void embed(const int32_t* tok, const uint16_t* table, int T, int H, int V, float* h,
           hipStream_t s) {
  hipLaunchKernelGGL(embed_k, dim3(T), dim3(256), 0, s, tok, table, H, V, h);
}
void lse_chunk(const float* logits, int T, int Vc, int v0, const int32_t* tgt, float* run_m,
               float* run_s, float* tlogit, int first, hipStream_t s) {
  hipLaunchKernelGGL(lse_chunk_k<false>, dim3(T), dim3(256), 0, s, logits, Vc, v0, tgt, run_m,
                     run_s, tlogit, nullptr, nullptr, first);
}
void lse_final(const float* run_m, const float* run_s, const float* tlogit, const int32_t* tgt,
               int T, int V, float* logp, float* lse, float* inv, hipStream_t s) {
  hipLaunchKernelGGL(lse_final_k, dim3(nb(T, 256)), dim3(256), 0, s, run_m, run_s, tlogit, tgt, T,
                     V, logp, lse, inv);
}
void lse_chunk_acc(const float* logits, int T, int Vc, int v0, const int32_t* tgt, float* run_m,
                   float* run_s, float* tlogit, float* alpha, uint16_t* pt, int first,
                   hipStream_t s) {
  hipLaunchKernelGGL(lse_chunk_k<true>, dim3(T), dim3(256), 0, s, logits, Vc, v0, tgt, run_m,
                     run_s, tlogit, alpha, pt, first);
}
void scale_rows(float* x, const float* f, int T, int n, hipStream_t s) {
  if (n % 4 == 0 && ((uintptr_t)x & 15) == 0) {
    const int64_t total4 = (int64_t)T * n / 4;
    hipLaunchKernelGGL(scale_rows_k, dim3(nb(total4, 256)), dim3(256), 0, s,
                       reinterpret_cast<f32x4*>(x), f, n / 4, total4);
  } else {
    const int64_t total = (int64_t)T * n;
    hipLaunchKernelGGL(scale_rows1_k, dim3(nb(total, 256)), dim3(256), 0, s, x, f, n, total);
  }
}
void head_grad(const float* dlogp, const int32_t* tgt, const uint16_t* W, int T, int H, int V,
               float* E, hipStream_t s) {
  const int64_t n = (int64_t)T * H;
  hipLaunchKernelGGL(head_grad_k, dim3(nb(n, 256)), dim3(256), 0, s, dlogp, tgt, W, H, V, n, E);
}
void sft_loss(const float* logp, const int32_t* tgt, int n, float* loss, float* dlogp,
              hipStream_t s) {
  hipLaunchKernelGGL(sft_loss_k, dim3(1), dim3(1024), 0, s, logp, tgt, n, loss, dlogp);
}
void pref_loss(int kind, const float* lp, const float* lr, int S, int P, float beta, float p2,
               float* out, float* dlogp, hipStream_t s) {
  hipLaunchKernelGGL(pref_loss_k, dim3(1), dim3(1024), 0, s, kind, lp, lr, S, P, beta, p2, out,
                     dlogp);
}
void sgd(float* p, const float* g, float lr, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(sgd_k, dim3(nb(n, 256)), dim3(256), 0, s, p, g, lr, n);
}
void group_sum(const float* part, int n_seq, int nq, int grp, int S, int d, float* out,
               int64_t ldo, hipStream_t s) {
  const int64_t total4 = (int64_t)n_seq * (nq / grp) * S * (d / 4);
  hipLaunchKernelGGL(group_sum4_k, dim3(nb(total4, 256)), dim3(256), 0, s,
                     reinterpret_cast<const f32x4*>(part), nq, grp, S, d / 4, out, ldo, total4);
}
void spin_us(uint32_t us, int wall_khz, hipStream_t s) {
  const uint64_t ticks = (uint64_t)us * (uint64_t)wall_khz / 1000u;
  hipLaunchKernelGGL(spin_k, dim3(1), dim3(64), 0, s, ticks);
}
void fill_u32(void* p, uint32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(fill_k, dim3(nb(n, 256)), dim3(256), 0, s, (uint32_t*)p, v, n);
}
void f32_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t s) {
  if (n % 4 == 0 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)y & 7) == 0)
    hipLaunchKernelGGL(f32_to_bf16_x4_k, dim3(nb(n / 4, 256)), dim3(256), 0, s,
                       reinterpret_cast<const f32x4*>(x), reinterpret_cast<u32x2*>(y), n / 4);
  else
    hipLaunchKernelGGL(f32_to_bf16_k, dim3(nb(n, 256)), dim3(256), 0, s, x, y, n);
}
void nf4_dequant(const uint8_t* codes, const float* absmax, int64_t n, const float* levels,
                 float* of32, uint16_t* obf, hipStream_t s) {
  Levels lv;
  for (int i = 0; i < 16; ++i) lv.v[i] = levels[i];
  const int64_t nw = n / 8;
  hipLaunchKernelGGL(nf4_dequant_k, dim3(nb(nw, 256)), dim3(256), 0, s, (const uint32_t*)codes,
                     absmax, nw, lv, of32, (u32x4*)obf);
}

}  // namespace lsn
