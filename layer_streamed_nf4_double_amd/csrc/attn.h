// Fused causal grouped-query attention forward (attn.hip).
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

// shapes the fused kernel takes: d 64 or 128, S a multiple of 64 up to 512
bool attn_fwd_ok(int S, int d, int64_t ld, int64_t ldo, const void* qkv, const void* O,
                 const void* frag);
// writes the fragment-ordered operands, then runs the fused kernel (grid
// S/64 x n_seq nq)
hipError_t attn_fwd(const AttnFwdParams& p, int d, hipStream_t s);

}  // namespace lsn
