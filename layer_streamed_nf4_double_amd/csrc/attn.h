// Fused causal grouped-query attention (attn.hip): the forward, and the
// query side of the backward (dS and dQ).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsn {

struct AttnFwdParams {
  const uint16_t* qkv;  // [T, ld] bf16 rows: q (nq d, roped) | k (nkv d, roped) | v (nkv d)
  int64_t ld;
  uint16_t* frag;       // scratch, T (nq + 2 nkv) d bf16: fragment-ordered q, k, v^T
  uint16_t* O;          // [T, ldo] bf16: head h at columns h d
  int64_t ldo;
  float* Pf;            // null, or [n_seq][nq][S][S]: P (fp32) for the keys of each query's tile
  uint16_t* Pb;         // null, or [n_seq][nq][S][S]: P (bf16), zero above the diagonal
  int n_seq, S, nq, nkv;
  float alpha;          // score scale 1/sqrt(d)
};

// dP = dO v^T, dS = P (dP - rowsum(P dP)), dQ = alpha dS k
struct AttnBwdParams {
  const uint16_t* qkv;  // [T, ld] bf16 rows as the forward's (k and v are read)
  int64_t ld;
  const uint16_t* dO;   // [T, lddo] bf16: gradient of the attention output
  int64_t lddo;
  uint16_t* frag;       // scratch, T (nq + 2 nkv) d bf16: fragment-ordered dO, v, k^T
  const float* Pin;     // [n_seq][nq][S][S]: P (fp32) as the forward wrote it
  uint16_t* dS;         // [n_seq][nq][S][S] bf16: dS, zero above the diagonal
  float* dQ;            // [T, ldq] fp32: head h at columns h d
  int64_t ldq;
  int n_seq, S, nq, nkv;
  float alpha;
};

// shapes the fused kernels take: d 64 or 128, S a multiple of 64 up to 512
bool attn_fwd_ok(int S, int d, int64_t ld, int64_t ldo, const void* qkv, const void* O,
                 const void* frag);
bool attn_bwd_ok(int S, int d, int64_t ld, int64_t lddo, int64_t ldq, const void* qkv,
                 const void* dO, const void* dQ, const void* frag, const void* Pin);
// each writes its fragment-ordered operands, then runs the fused kernel
// (grid S/64 x n_seq nq)
hipError_t attn_fwd(const AttnFwdParams& p, int d, hipStream_t s);
hipError_t attn_bwd(const AttnBwdParams& p, int d, hipStream_t s);

}  // namespace lsn
