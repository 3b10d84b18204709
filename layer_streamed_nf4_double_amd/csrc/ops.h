// Launchers of the per-layer kernels (ops.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsn {
// An fp32 operand [rows, width] given as the sum of ns buffers p + y stride
// (y < ns, rows of the operand's own width): the split-k partial sums of the
// GEMM that produced it, which a consumer adds in split order exactly as the
// split-k reduction would (ns = 1: the operand itself).  The *_fuses checks
// say whether a consumer takes ns > 1 (16-byte aligned p and stride % 4 == 0
// also required); otherwise it needs ns = 1.
struct SplitSum {
  const float* p = nullptr;
  int ns = 1;
  int64_t stride = 0;
};
bool rmsnorm_bwd_fuses(int H, const float* h, const float* out, const float* dres,
                       const uint16_t* g);
// outb (may be null): also bf16(out)
void rmsnorm_bwd(const float* h, const uint16_t* g, const float* rstd, const SplitSum& dy,
                 const float* dres, int T, int H, float* out, uint16_t* outb, hipStream_t s);
// hout = res + src, then y = RMSNorm(hout) (needs rmsnorm_fwd_res_fuses)
bool rmsnorm_fwd_res_fuses(int H, const float* res, const float* hout, const uint16_t* g,
                           const uint16_t* y);
void rmsnorm_fwd_res(const float* res, const SplitSum& src, const uint16_t* g, int T, int H,
                     float eps, float* hout, uint16_t* y, float* rstd, hipStream_t s);
bool rope_fwd_fuses(int d, const uint16_t* out);
void rope_fwd(const SplitSum& qkv, uint16_t* out, int T, int S, int nq, int nkv, int d,
              float theta, hipStream_t s);
bool swiglu_bwd_fuses(int T, int F, const float* gu, const uint16_t* dgu, const float* dguf);
void swiglu_bwd(const float* gu, const SplitSum& da, uint16_t* dgu, float* dguf, int T, int F,
                hipStream_t s);
void rmsnorm_fwd(const float* h, const uint16_t* g, int T, int H, float eps, uint16_t* y,
                 float* rstd, hipStream_t s);
void rmsnorm_bwd(const float* h, const uint16_t* g, const float* rstd, const float* dy,
                 const float* dres, int T, int H, float* out, hipStream_t s);
void rope_fwd(const float* qkv, uint16_t* out, int T, int S, int nq, int nkv, int d, float theta,
              hipStream_t s);
void rope_bwd(float* dqkv, uint16_t* outb, int T, int S, int nq, int nkv, int d, float theta,
              hipStream_t s);
void softmax_causal(const float* sc, float* Pf, uint16_t* Pb, int S, int64_t rows, hipStream_t s);
void softmax_bwd(const float* Pf, const float* dP, uint16_t* dS, int S, int64_t rows,
                 hipStream_t s);
void swiglu_fwd(const float* gu, uint16_t* a, int T, int F, hipStream_t s);
void swiglu_bwd(const float* gu, const float* da, uint16_t* dgu, float* dguf, int T, int F,
                hipStream_t s);
void embed(const int32_t* tok, const uint16_t* table, int T, int H, int V, float* h,
           hipStream_t s);
void lse_chunk(const float* logits, int T, int Vc, int v0, const int32_t* tgt, float* run_m,
               float* run_s, float* tlogit, int first, hipStream_t s);
// targets >= V give NaN log-probs (no vocabulary entry), negative ones 0
void lse_final(const float* run_m, const float* run_s, const float* tlogit, const int32_t* tgt,
               int T, int V, float* logp, float* lse, float* inv, hipStream_t s);
// chunk pass that also writes p~ = bf16(exp(l - m')) and alpha = exp(m - m')
void lse_chunk_acc(const float* logits, int T, int Vc, int v0, const int32_t* tgt, float* run_m,
                   float* run_s, float* tlogit, float* alpha, uint16_t* pt, int first,
                   hipStream_t s);
// x[t, :] *= f[t] (n % 4 == 0, 16-byte aligned rows)
void scale_rows(float* x, const float* f, int T, int n, hipStream_t s);
// E[t, :] = dlogp[t] * (W[y_t, :] - E[t, :]) in place (W[y_t] taken as 0
// for y_t outside [0, V))
void head_grad(const float* dlogp, const int32_t* tgt, const uint16_t* W, int T, int H, int V,
               float* E, hipStream_t s);
void sft_loss(const float* logp, const int32_t* tgt, int n, float* loss, float* dlogp,
              hipStream_t s);
// kind: 0 DPO, 1 SimPO, 2 ORPO, 3 KTO (lr may be null for 1 and 2)
void pref_loss(int kind, const float* lp, const float* lr, int S, int P, float beta, float p2,
               float* out, float* dlogp, hipStream_t s);
void sgd(float* p, const float* g, float lr, int64_t n, hipStream_t s);
// out[(q S + i) ldo + kv d + j] = sum over the grp q heads of kv (head
// order) of part[((q nq + h) S + i) d + j]; d % 4 == 0, 16-byte aligned rows
void group_sum(const float* part, int n_seq, int nq, int grp, int S, int d, float* out,
               int64_t ldo, hipStream_t s);
// a kernel that waits `us` microseconds of the device wall clock (rate
// wall_khz) on stream s, then exits
void spin_us(uint32_t us, int wall_khz, hipStream_t s);
void fill_u32(void* p, uint32_t v, int64_t n, hipStream_t s);
void f32_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t s);
void nf4_dequant(const uint8_t* codes, const float* absmax, int64_t n, const float* levels,
                 float* of32, uint16_t* obf, hipStream_t s);
}  // namespace lsn
