// liblsn runtime: context, workspace carving, pinned host store, the
// double-buffered layer stream scheduler, layer orchestration and the C ABI.
//
// The mechanism ("Soup: Fine-Tune an 8B Model on a 4 GB GPU", section "The Core
// Idea: Layer Streaming"): the frozen base stays in host RAM (here: one pinned
// arena, or a file) and is copied to the GPU one decoder layer at a time, on a
// dedicated stream, as the forward or backward pass reaches it.  Here each
// layer is one contiguous record (NF4 codes of the seven projections, their
// absmax scales, the two norm gains); two device slots alternate, so the copy
// of layer i+1 runs on the copy stream while layer i computes.  Events order
// the streams: the compute stream waits for copy_done[slot] before a layer,
// and the copy into a slot waits for slot_free[slot] recorded after the
// slot's previous layer finished.  A record already sitting in a slot when a
// pass reaches it (the last two layers of a forward pass are the first two of
// the backward pass) is reused instead of copied again.
//
// The slot bookkeeping (which record goes into which slot, which event each
// stream waits for) is the SlotScheduler of sched.h; this file supplies its
// executor (HIP stream operations) and the record sources.
//
// Resident mode keeps every record in device memory at the same intra-record
// offsets, so the kernels run on byte-identical inputs: streamed and resident
// results are bit-identical (the pages' own correctness bar, axbrief.com
// article, "Beyond Memory: The Layer Streaming Breakthrough").
#include <errno.h>
#include <fcntl.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>
#include <sys/mman.h>
#include <unistd.h>

#include <algorithm>
#include <condition_variable>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/lsn.h"
#include "attn.h"
#include "gemm.h"
#include "host_codec.h"
#include "lora.h"
#include "ops.h"
#include "sched.h"

using namespace lsn;

namespace {

constexpr int NPROJ = 7;
constexpr uint64_t REC_ALIGN = 4096;
// Vocabulary rows per LM-head GEMM: about 256 output tiles of 256 x 256 at
// max_tokens rows (one workgroup per CU, no split-k), at least 16384.  The
// fp32 logits of one chunk then take at most 64 MiB up to 1024 tokens.
inline int vchunk_for(int64_t max_tokens) {
  const int64_t mt = (max_tokens + 255) / 256;
  return (int)std::max<int64_t>(16384, std::min<int64_t>(65536, 256 / mt * 256));
}

inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

struct Carver {
  uint64_t off = 0;
  uint64_t take(uint64_t bytes) {
    off = align_up(off, 256);
    const uint64_t o = off;
    off += bytes;
    return o;
  }
};

}  // namespace

// The scheduler's executor: HIP stream operations on the context's streams
// (defined after lsn_ctx).
struct HipExec {
  lsn_ctx* c;
  int copy_wait_free(int s);
  int host_wait_copy(int s);
  int copy_record(int layer, int s, int next);
  int compute_wait_copy(int s);
  int compute_free(int s);
};

struct lsn_ctx {
  lsn_config cfg{};
  std::string store_path;
  hipStream_t cs = nullptr;    // compute stream (caller's)
  hipStream_t copy = nullptr;  // the scheduler's copy stream
  hipEvent_t copy_done[MAX_SLOTS] = {};
  hipEvent_t slot_free[MAX_SLOTS] = {};
  SlotScheduler<HipExec> sched;  // slots, pass order and position (streamed modes)
  int nslots = 2;
  int device = 0;

  char* ws = nullptr;
  uint64_t ws_bytes = 0, ws_needed = 0;

  // record layout
  int64_t N[NPROJ] = {}, K[NPROJ] = {};
  uint64_t code_off[NPROJ] = {}, amax_off[NPROJ] = {}, norm_off[2] = {};
  uint64_t rec_bytes = 0;
  int QKV = 0, QD = 0, KVD = 0;

  // host store
  uint8_t* store = nullptr;  // pinned, n_layers records (host / resident modes)
  uint8_t* bounce[MAX_SLOTS] = {};  // pinned bounce buffers, one per slot (file mode)
  int fd = -1;   // file mode: the store file, buffered (writes; reads without O_DIRECT)
  int dfd = -1;  // file mode: the same file opened O_DIRECT for the record reads
  // File mode: a reader thread fills two page-aligned staging buffers, each
  // tagged with the layer it holds.  The host thread takes a staged record,
  // asks for the next record of the pass in the other buffer, and copies the
  // staged one into the slot's pinned bounce buffer meanwhile.
  struct Reader {
    std::thread th;
    std::mutex mu;
    std::condition_variable cv;
    uint8_t* buf[2] = {nullptr, nullptr};
    int layer[2] = {-1, -1};  // record held or being read (-1: none)
    bool ready[2] = {false, false};
    int err[2] = {0, 0};      // errno of a failed read (EIO for a short file)
    int req = -1;             // buffer the thread fills next (-1: none)
    bool quit = false;
  } rd;
  std::vector<char> loaded;

  // device regions
  uint8_t* records = nullptr;  // resident: L records; streamed: 2 slots
  // embed / lm_head: device tables, or with head_on_host device-visible
  // pointers to the pinned host copies embed_h / lm_head_h
  uint16_t *embed = nullptr, *lm_head = nullptr, *final_norm = nullptr;
  uint16_t *embed_h = nullptr, *lm_head_h = nullptr;
  float *lora_p = nullptr, *lora_g = nullptr;
  uint64_t lora_n = 0;
  std::vector<int64_t> lA, lB;  // float offsets of A and B per (layer, proj); -1 if none
  bool head_loaded = false;

  // activation scratch (one layer at TL tokens)
  uint16_t *n1, *qkvb, *Pb, *O, *n2, *a, *dgu, *dO, *dqkvb, *aext, *bext, *nf, *dlog;
  float *rstd1, *qkv, *scores, *Pf, *h2, *rstd2, *gu, *da, *dguf, *dn, *dh2, *dqkv, *lt, *lu,
      *rstdf, *logits, *run_m, *run_s, *tlogit, *lse, *dnf, *lpart, *gpart, *hpart;
  int64_t ext_rows = 0, lpart_floats = 0, gpart_floats = 0;
  int vchunk = 16384;  // vocabulary rows per LM-head GEMM (vchunk_for(max_tokens))

  // pass state (the layer order and position live in sched)
  int pass_kind = -1, n_seq = 0, seq_len = 0, T = 0;
  int64_t TL = 0;  // tokens the layer workspace holds (layer_tokens, else max_tokens)
  bool adapters_on = true;
  const float* lm_h = nullptr;
  int lm_T = 0;
  bool lm_grad = false;  // the last lm_head_logprobs kept the expected-row accumulator
  // forward B extensions (bf16 block layout of B_p^T), one per layer and
  // adapted group, valid while fext_ver matches lora_version (bumped by every
  // adapter write)
  uint16_t* fext = nullptr;
  std::vector<int64_t> fext_off;
  uint16_t* fat = nullptr;            // bf16(A_p)^T [16, K_p] per layer and adapter
  std::vector<int64_t> fat_off;
  std::vector<uint64_t> fext_ver;
  uint64_t lora_version = 1;
  const uint16_t* fwd_bext = nullptr;  // the extension of the group being launched
  float* head_f = nullptr;  // per-row factors of the LM head [T]

  float levels[16];
  uint64_t bytes_h2d = 0;
  // fault injection (tests): spin on the copy stream before each slot copy,
  // spin on the compute stream before each layer's kernels, fill a slot with
  // NaN bytes before each copy into it
  uint32_t copy_delay_us = 0, compute_delay_us = 0;
  bool poison_slots = false;
  int wall_khz = 100000;  // device wall-clock rate for the spins

  // optional timing of GEMM launches and record copies (event pairs)
  struct ProfRec {
    int what, a, b, tile;
    double work;
    hipEvent_t e0, e1;
  };
  int profiling = 0;  // bit 0: NF4 GEMM launches, bit 1: record copies
  std::vector<ProfRec> prof;
  std::vector<hipEvent_t> evpool;
  size_t evnext = 0;
  bool poisoned = false;
  std::string err;

  bool targeted(int p) const { return (cfg.lora_targets >> p) & 1u; }
  float lora_scale() const { return cfg.lora_alpha / (float)cfg.lora_rank; }
  float* A_of(int layer, int p) const {
    const int64_t o = lA[layer * NPROJ + p];
    return o < 0 ? nullptr : lora_p + o;
  }
  float* B_of(int layer, int p) const {
    const int64_t o = lB[layer * NPROJ + p];
    return o < 0 ? nullptr : lora_p + o;
  }
  float* dA_of(int layer, int p) const {
    const int64_t o = lA[layer * NPROJ + p];
    return o < 0 ? nullptr : lora_g + o;
  }
  float* dB_of(int layer, int p) const {
    const int64_t o = lB[layer * NPROJ + p];
    return o < 0 ? nullptr : lora_g + o;
  }
};

// ---------------------------------------------------------------------------
// error plumbing
// ---------------------------------------------------------------------------
static lsn_status fail(lsn_ctx* c, lsn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c) {
    c->err = buf;
    if (st == LSN_ERR_HIP || st == LSN_ERR_IO) c->poisoned = true;
  }
  return st;
}

#define HIPCHK(c, expr)                                                                     \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess)                                                                   \
      return fail(c, LSN_ERR_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), \
                  __FILE__, __LINE__);                                                      \
  } while (0)

// hipGetLastError reports the last failed HIP call of the thread, whoever
// made it; a status left by the caller's own HIP calls (a not-ready event or
// stream query, say) is theirs, so every entry point clears it first and the
// launch checks see only this call's errors.
#define CHECK_CTX(c)                                                  \
  do {                                                                \
    if (!(c)) return LSN_ERR_INVALID;                                 \
    if ((c)->poisoned) return LSN_ERR_STATE;                          \
    (void)hipGetLastError();                                          \
  } while (0)

// Calls without a context keep their last error message per thread
// (lsn_last_error(NULL)).
static thread_local std::string g_err;

static lsn_status fail0(lsn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

// the status of the launches of a call without a context
static lsn_status launch_status0(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return LSN_OK;
  return fail0(LSN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static lsn_status launch_check(lsn_ctx* c) {
  HIPCHK(c, hipGetLastError());
  return LSN_OK;
}

// ---------------------------------------------------------------------------
// profiling
// ---------------------------------------------------------------------------
// Timing events only bracket work for elapsed-time queries made after a full
// synchronization, so they skip the system-scope fence of an event record
// (an L2 writeback that would itself take time between the brackets).
static hipEvent_t take_event(lsn_ctx* c) {
  if (c->evnext == c->evpool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    c->evpool.push_back(e);
  }
  return c->evpool[c->evnext++];
}

static bool prof_begin(lsn_ctx* c, lsn_ctx::ProfRec* r, hipStream_t s) {
  if (!(c->profiling & 2)) return false;
  r->e0 = take_event(c);
  r->e1 = take_event(c);
  if (!r->e0 || !r->e1) return false;
  return hipEventRecord(r->e0, s) == hipSuccess;
}

static void prof_end(lsn_ctx* c, lsn_ctx::ProfRec& r, hipStream_t s) {
  if (hipEventRecord(r.e1, s) == hipSuccess) c->prof.push_back(r);
}

// every GEMM of a context goes through here; the NF4 ones can be timed
// keep (may be null): when the launch splits k, its partial sums stay in
// gpart for the next kernel, which adds them (*keep describes them; else
// *keep is the output itself)
static hipError_t cgemm(lsn_ctx* c, GemmParams p, int opa, int opb, int batch,
                        SplitSum* keep = nullptr) {
  p.part = c->gpart;
  p.part_floats = c->gpart_floats;
  int ns = 1;
  if (keep) {
    p.defer_reduce = 1;
    p.split_used = &ns;
  }
  lsn_ctx::ProfRec r{0, opa, opb, gemm_tile(p, opa, opb, batch),
                     2.0 * p.M * p.N * (double)p.K * p.nseg * batch, nullptr, nullptr};
  // events bracket the GEMM kernel only (not a split-k reduction)
  const bool on = (c->profiling & 1) && (opb == B_NF4_K || opb == B_NF4_R);
  if (on) {
    r.e0 = take_event(c);
    r.e1 = take_event(c);
    p.ev0 = r.e0;
    p.ev1 = r.e1;
  }
  const hipError_t e = gemm(p, opa, opb, batch, c->cs);
  if (on && r.e0 && r.e1) c->prof.push_back(r);
  if (keep)
    *keep = ns > 1 ? SplitSum{c->gpart, ns, split_stride(p.M, p.N)}
                   : SplitSum{static_cast<const float*>(p.C), 1, 0};
  return e;
}

// ---------------------------------------------------------------------------
// configuration checks and layout
// ---------------------------------------------------------------------------
static bool cfg_valid(const lsn_config* g, std::string* why) {
  auto bad = [&](const char* m) {
    *why = m;
    return false;
  };
  if (!g) return bad("null config");
  if (g->n_layers <= 0 || g->hidden <= 0 || g->n_heads <= 0 || g->n_kv_heads <= 0 ||
      g->head_dim <= 0 || g->ffn <= 0 || g->vocab <= 0)
    return bad("non-positive shape");
  if (g->n_heads % g->n_kv_heads) return bad("n_heads must be a multiple of n_kv_heads");
  if (g->head_dim % 16) return bad("head_dim must be a multiple of 16");
  if (g->hidden % 16 || g->ffn % 16) return bad("hidden and ffn must be multiples of 16");
  if (g->vocab % 8) return bad("vocab must be a multiple of 8");
  if (g->lora_rank < 1 || g->lora_rank > 16) return bad("lora_rank must be 1..16");
  if (g->lora_targets >= (1u << NPROJ)) return bad("lora_targets has unknown bits");
  if (g->max_tokens <= 0 || g->max_seq_len <= 0 || g->max_seq_len > g->max_tokens)
    return bad("bad max_tokens / max_seq_len");
  if (g->mode < LSN_RESIDENT || g->mode > LSN_STREAM_FILE) return bad("bad mode");
  if (g->mode == LSN_STREAM_FILE && (!g->store_path || !g->store_path[0]))
    return bad("file mode needs store_path");
  if (!(g->rms_eps > 0.f) || !(g->rope_theta > 0.f)) return bad("bad eps / theta");
  if (g->head_on_host && g->mode == LSN_RESIDENT)
    return bad("head_on_host needs a streamed base (the head streams through its slots)");
  if (g->head_chunk_rows < 0 || g->head_chunk_rows % 8) return bad("head_chunk_rows must be a multiple of 8");
  if (g->n_slots != 0 && (g->n_slots < 2 || g->n_slots > MAX_SLOTS))
    return bad("n_slots must be 0 (two) or 2..4");
  if (g->layer_tokens < 0) return bad("layer_tokens must be >= 0");
  return true;
}

// device slots of a streamed configuration (0 in the config: a double buffer)
static int slot_count(const lsn_config* g) { return g->n_slots ? g->n_slots : 2; }

// Vocabulary rows per LM-head chunk: the configured count, else
// vchunk_for(max_tokens), and with head_on_host (W_lm streams through the
// layer slots) no more rows than one slot holds, rounded down to a multiple
// of 256 (of 8 for a slot of fewer than 256 rows).
static int head_chunk_rows(const lsn_ctx* c) {
  const lsn_config& g = c->cfg;
  if (g.head_chunk_rows > 0) return g.head_chunk_rows;
  int64_t v = vchunk_for(g.max_tokens);
  if (g.head_on_host) {
    const int64_t slot_rows = (int64_t)(c->rec_bytes / ((uint64_t)g.hidden * 2));
    v = std::min<int64_t>(v, slot_rows >= 256 ? slot_rows / 256 * 256 : slot_rows / 8 * 8);
  }
  return (int)v;
}

// Checks that need the record layout: a head chunk must fit a slot.
static bool layout_valid(const lsn_ctx* c, std::string* why) {
  const lsn_config& g = c->cfg;
  const int64_t rows = head_chunk_rows(c);
  if (g.head_on_host && (rows < 8 || (uint64_t)rows * g.hidden * 2 > c->rec_bytes)) {
    *why = "an LM-head chunk of W_lm rows must fit one layer slot";
    return false;
  }
  return true;
}

static void record_layout(lsn_ctx* c) {
  const lsn_config& g = c->cfg;
  const int64_t H = g.hidden, F = g.ffn;
  c->QD = g.n_heads * g.head_dim;
  c->KVD = g.n_kv_heads * g.head_dim;
  c->QKV = c->QD + 2 * c->KVD;
  const int64_t n[NPROJ] = {c->QD, c->KVD, c->KVD, H, F, F, H};
  const int64_t k[NPROJ] = {H, H, H, c->QD, H, H, F};
  uint64_t off = 0;
  for (int p = 0; p < NPROJ; ++p) {  // codes back to back (q|k|v and gate|up fuse)
    c->N[p] = n[p];
    c->K[p] = k[p];
    c->code_off[p] = off;
    off += (uint64_t)n[p] * k[p] / 2;
  }
  off = align_up(off, 256);
  for (int p = 0; p < NPROJ; ++p) {  // absmax back to back, same order
    c->amax_off[p] = off;
    off += (uint64_t)n[p] * k[p] / 64 * 4;
  }
  off = align_up(off, 256);
  c->norm_off[0] = off;
  off += H * 2;
  c->norm_off[1] = off;
  off += H * 2;
  c->rec_bytes = align_up(off, REC_ALIGN);
}

struct Group {
  int first, count;
};
static const Group G_QKV{LSN_Q, 3}, G_O{LSN_O, 1}, G_GU{LSN_GATE, 2}, G_D{LSN_DOWN, 1};
// a group's adapter conversions (two per adapter) fit one batch
constexpr int MAX_GROUP = 3;
static_assert(2 * MAX_GROUP <= (int)(sizeof(ExtBatch::job) / sizeof(ExtJob)),
              "one conversion launch per group");

static int64_t group_rows(const lsn_ctx* c, Group g) {
  int64_t n = 0;
  for (int p = g.first; p < g.first + g.count; ++p) n += c->N[p];
  return n;
}

// Carves the workspace; with base == nullptr only measures.
static uint64_t carve(lsn_ctx* c, char* base) {
  const lsn_config& g = c->cfg;
  const int64_t TH = g.max_tokens, S = g.max_seq_len, H = g.hidden, F = g.ffn, V = g.vocab;
  const int64_t r = g.lora_rank;
  // the layer buffers hold TL tokens (one group of whole sequences), the LM
  // head's hold TH (all tokens of a pass)
  const int64_t T = g.layer_tokens > 0
                        ? std::min<int64_t>(TH, std::max<int64_t>(g.layer_tokens, S))
                        : TH;
  c->TL = T;
  c->vchunk = head_chunk_rows(c);
  Carver cv;
  auto P = [&](uint64_t bytes) -> char* { const uint64_t o = cv.take(bytes); return base ? base + o : nullptr; };
  const int nrec = (g.mode == LSN_RESIDENT) ? g.n_layers : slot_count(&g);
  c->records = (uint8_t*)P((uint64_t)nrec * c->rec_bytes);
  if (!g.head_on_host) {
    c->embed = (uint16_t*)P(V * H * 2);
    c->lm_head = g.tied_embeddings ? c->embed : (uint16_t*)P(V * H * 2);
  }
  c->final_norm = (uint16_t*)P(H * 2);
  // adapters
  c->lA.assign((size_t)g.n_layers * NPROJ, -1);
  c->lB.assign((size_t)g.n_layers * NPROJ, -1);
  uint64_t nfl = 0;
  for (int l = 0; l < g.n_layers; ++l)
    for (int p = 0; p < NPROJ; ++p)
      if (c->targeted(p)) {
        c->lA[l * NPROJ + p] = (int64_t)nfl;
        nfl += align_up((uint64_t)c->K[p] * r, 64);
        c->lB[l * NPROJ + p] = (int64_t)nfl;
        nfl += align_up((uint64_t)r * c->N[p], 64);
      }
  c->lora_n = nfl;
  c->lora_p = (float*)P(std::max<uint64_t>(nfl, 1) * 4);
  c->lora_g = (float*)P(std::max<uint64_t>(nfl, 1) * 4);
  // one layer of activations
  const int64_t Z = (int64_t)g.n_heads * T * S;  // sum over sequences of heads * S * S
  const int64_t QKV = c->QKV, QD = c->QD;
  c->n1 = (uint16_t*)P(T * H * 2);
  c->rstd1 = (float*)P(T * 4);
  c->qkv = (float*)P(T * QKV * 4);
  c->qkvb = (uint16_t*)P(T * QKV * 2);
  c->scores = (float*)P(Z * 4);
  c->Pf = (float*)P(Z * 4);
  c->Pb = (uint16_t*)P(Z * 2);
  c->O = (uint16_t*)P(T * QD * 2);
  c->h2 = (float*)P(T * H * 4);
  c->n2 = (uint16_t*)P(T * H * 2);
  c->rstd2 = (float*)P(T * 4);
  c->gu = (float*)P(T * 2 * F * 4);
  c->a = (uint16_t*)P(T * F * 2);
  c->da = (float*)P(T * F * 4);
  c->dgu = (uint16_t*)P(T * 2 * F * 2);
  c->dguf = (float*)P(T * 2 * F * 4);
  c->dn = (float*)P(T * H * 4);
  c->dh2 = (float*)P(T * H * 4);
  c->dO = (uint16_t*)P(T * QD * 2);
  c->dqkv = (float*)P(T * QKV * 4);
  // bf16 q|k|v input gradient, and the bf16 copy of the fp32 output gradient
  // [T, hidden] that the dX GEMMs of down and o take: the larger of the two
  c->dqkvb = (uint16_t*)P(T * std::max<int64_t>(QKV, H) * 2);
  c->hpart = (float*)P(T * QD * 4);  // per-q-head dV / dK before the group sum
  c->lt = (float*)P(NPROJ * T * 16 * 4);
  // the down-projections' split sums (any token count up to T)
  c->lpart_floats = lora_down_partial_floats_max((int)T, 3);
  for (int p = 0; p < NPROJ; ++p)
    if (c->targeted(p))
      c->lpart_floats = std::max<int64_t>(
          {c->lpart_floats, lora_mm_partial_floats((int)T, (int)c->K[p]),
           lora_mm_partial_floats((int)T, (int)c->N[p]), lora_mm_partial_floats((int)c->K[p], (int)T),
           lora_mm_partial_floats((int)c->N[p], (int)T)});
  c->lpart = (float*)P(std::max<int64_t>(c->lpart_floats, 1) * 4);
  {  // split-k scratch of the largest single-problem GEMM: a layer's at TL
     // tokens, the LM head's at max_tokens
    const int64_t Vc0 = std::min<int64_t>(V, c->vchunk);
    const int64_t shapes[][3] = {{QKV, H, T},  {H, QD, T},  {2 * F, H, T}, {H, F, T},
                                 {F, H, T},    {H, 2 * F, T}, {QD, H, T},  {H, QKV, T},
                                 {Vc0, H, TH}, {H, Vc0, TH}};
    c->gpart_floats = 0;
    for (const auto& sh : shapes)
      c->gpart_floats = std::max<int64_t>(
          c->gpart_floats, gemm_partial_floats((int)sh[2], (int)sh[0], (int)sh[1], 1, 1));
    c->gpart = (float*)P(std::max<int64_t>(c->gpart_floats, 1) * 4);
  }
  c->lu = (float*)P(3 * T * 16 * 4);  // u_p of up to three adapters of a group
  c->ext_rows = std::max<int64_t>({QKV, 2 * F, H, QD, F});
  c->aext = (uint16_t*)P(T * 48 * 2);
  c->bext = (uint16_t*)P(c->ext_rows * 48 * 2);
  {
    const Group groups[4] = {G_QKV, G_O, G_GU, G_D};
    c->fext_off.assign((size_t)g.n_layers * 4, -1);
    c->fext_ver.assign((size_t)g.n_layers * 4, 0);
    uint64_t fe = 0;
    for (int l = 0; l < g.n_layers; ++l)
      for (int gi = 0; gi < 4; ++gi) {
        int nad = 0;
        for (int p = groups[gi].first; p < groups[gi].first + groups[gi].count; ++p)
          nad += c->targeted(p);
        if (!nad) continue;
        c->fext_off[(size_t)l * 4 + gi] = (int64_t)fe;
        fe += align_up((uint64_t)group_rows(c, groups[gi]) * 16 * nad, 128);
      }
    c->fext = (uint16_t*)P(std::max<uint64_t>(fe, 1) * 2);
    c->fat_off.assign((size_t)g.n_layers * NPROJ, -1);
    uint64_t fa = 0;
    for (int l = 0; l < g.n_layers; ++l)
      for (int p = 0; p < NPROJ; ++p)
        if (c->targeted(p)) {
          c->fat_off[(size_t)l * NPROJ + p] = (int64_t)fa;
          fa += align_up((uint64_t)16 * c->K[p], 64);
        }
    c->fat = (uint16_t*)P(std::max<uint64_t>(fa, 1) * 2);
  }
  // LM head
  const int64_t Vc = std::min<int64_t>(V, c->vchunk);
  c->nf = (uint16_t*)P(TH * H * 2);
  c->rstdf = (float*)P(TH * 4);
  c->logits = (float*)P(TH * Vc * 4);
  c->dlog = (uint16_t*)P(TH * Vc * 2);
  c->run_m = (float*)P(TH * 4);
  c->run_s = (float*)P(TH * 4);
  c->tlogit = (float*)P(TH * 4);
  c->lse = (float*)P(TH * 4);
  c->head_f = (float*)P(TH * 4);
  c->dnf = (float*)P(TH * H * 4);
  return align_up(cv.off, 256);
}

// ---------------------------------------------------------------------------
// scheduler
// ---------------------------------------------------------------------------
// dst = src for n bytes, split over a few threads (host memory to pinned
// host memory; one thread moves ~10 GB/s, a record is ~120 MB at 8B).
static void parallel_copy(uint8_t* dst, const uint8_t* src, uint64_t n) {
  constexpr int NT = 8;
  const uint64_t part = (n / NT + 4095) & ~(uint64_t)4095;
  std::thread th[NT - 1];
  int started = 0;
  for (int i = 1; i < NT; ++i) {
    const uint64_t b = (uint64_t)i * part;
    if (b >= n) break;
    const uint64_t len = std::min(part, n - b);
    th[started++] = std::thread([=] { memcpy(dst + b, src + b, len); });
  }
  memcpy(dst, src, std::min(part, n));
  for (int i = 0; i < started; ++i) th[i].join();
}

static int read_record(const lsn_ctx* c, uint8_t* dst, int layer) {
  const int fd = c->dfd >= 0 ? c->dfd : c->fd;
  const uint64_t off = (uint64_t)layer * c->rec_bytes;
  uint64_t done = 0;
  while (done < c->rec_bytes) {
    const ssize_t got = pread(fd, dst + done, c->rec_bytes - done, off + done);
    if (got < 0) return errno ? errno : EIO;
    if (got == 0) return EIO;
    done += (uint64_t)got;
  }
  return 0;
}

static void reader_main(lsn_ctx* c) {
  lsn_ctx::Reader& r = c->rd;
  std::unique_lock<std::mutex> lk(r.mu);
  for (;;) {
    r.cv.wait(lk, [&] { return r.quit || r.req >= 0; });
    if (r.quit) return;
    const int i = r.req, layer = r.layer[i];
    r.req = -1;
    lk.unlock();
    const int e = read_record(c, r.buf[i], layer);
    lk.lock();
    r.err[i] = e;
    r.ready[i] = true;
    r.cv.notify_all();
  }
}

// Waits until the reader has nothing queued or in flight.
static void reader_idle(lsn_ctx::Reader& r, std::unique_lock<std::mutex>& lk) {
  r.cv.wait(lk, [&] {
    return r.req < 0 && (r.layer[0] < 0 || r.ready[0]) && (r.layer[1] < 0 || r.ready[1]);
  });
}

// Staging buffer holding the record of `layer`, read now if it is neither
// staged nor on its way; then the next record `next` (-1: none) is queued
// into the other buffer.  Returns -1 after a failed read (errno in *err).
static int reader_take(lsn_ctx* c, int layer, int next, int* err) {
  lsn_ctx::Reader& r = c->rd;
  std::unique_lock<std::mutex> lk(r.mu);
  int i = r.layer[0] == layer ? 0 : r.layer[1] == layer ? 1 : -1;
  if (i < 0 || (r.ready[i] && r.err[i])) {
    reader_idle(r, lk);
    i = r.layer[0] == next ? 1 : 0;  // keep a staged `next`
    r.layer[i] = layer;
    r.ready[i] = false;
    r.req = i;
    r.cv.notify_all();
  }
  r.cv.wait(lk, [&] { return r.ready[i]; });
  if (r.err[i]) {
    *err = r.err[i];
    r.layer[i] = -1;
    return -1;
  }
  const int j = 1 - i;
  if (next >= 0 && next != layer && r.layer[j] != next) {
    reader_idle(r, lk);
    r.layer[j] = next;
    r.ready[j] = false;
    r.req = j;
    r.cv.notify_all();
  }
  return i;
}

// A rewritten record must not be served from a staging buffer.
static void reader_forget(lsn_ctx* c, int layer) {
  lsn_ctx::Reader& r = c->rd;
  if (!r.th.joinable()) return;
  std::unique_lock<std::mutex> lk(r.mu);
  reader_idle(r, lk);
  for (int i = 0; i < 2; ++i)
    if (r.layer[i] == layer) r.layer[i] = -1;
}

// Fault injection: the spin and the NaN fill are ordinary kernels on the
// stream they delay, so results must not change (tests).
static void inject_copy_faults(lsn_ctx* c, uint8_t* dst, uint64_t bytes) {
  if (c->poison_slots) fill_u32(dst, 0xFFFFFFFFu, (int64_t)(bytes / 4), c->copy);
  if (c->copy_delay_us) spin_us(c->copy_delay_us, c->wall_khz, c->copy);
}

int HipExec::copy_wait_free(int s) {
  HIPCHK(c, hipStreamWaitEvent(c->copy, c->slot_free[s], 0));
  return LSN_OK;
}

// The host waits for the previous copy into a slot before queueing the next,
// so at most one copy per slot is queued.  With a whole step of copies queued
// the runtime's copy queue fills: hipMemcpyAsync then blocks the host for
// milliseconds and later copies reach the engine late.  Every dependency of
// the waited copy is already enqueued.  (For the file source this also frees
// the slot's bounce buffer.)
int HipExec::host_wait_copy(int s) {
  HIPCHK(c, hipEventSynchronize(c->copy_done[s]));
  return LSN_OK;
}

int HipExec::copy_record(int layer, int s, int next) {
  uint8_t* dst = c->records + (uint64_t)s * c->rec_bytes;
  const uint8_t* src;
  if (c->cfg.mode == LSN_STREAM_FILE) {
    // O_DIRECT cannot target the pinned bounce buffers (the kernel cannot
    // pin driver-mapped pages for direct I/O), so reads land in ordinary
    // page-aligned staging buffers and are copied over by several threads
    // while the reader fetches the next record.
    int err = 0;
    const int i = reader_take(c, layer, next, &err);
    if (i < 0)
      return fail(c, LSN_ERR_IO, "read of layer %d record failed: %s", layer, strerror(err));
    parallel_copy(c->bounce[s], c->rd.buf[i], c->rec_bytes);
    src = c->bounce[s];
  } else {
    src = c->store + (uint64_t)layer * c->rec_bytes;
  }
  inject_copy_faults(c, dst, c->rec_bytes);
  lsn_ctx::ProfRec r{1, 0, 0, 0, (double)c->rec_bytes, nullptr, nullptr};
  const bool on = prof_begin(c, &r, c->copy);
  HIPCHK(c, hipMemcpyAsync(dst, src, c->rec_bytes, hipMemcpyHostToDevice, c->copy));
  if (on) prof_end(c, r, c->copy);
  HIPCHK(c, hipEventRecord(c->copy_done[s], c->copy));
  c->bytes_h2d += c->rec_bytes;
  return LSN_OK;
}

int HipExec::compute_wait_copy(int s) {
  HIPCHK(c, hipStreamWaitEvent(c->cs, c->copy_done[s], 0));
  return LSN_OK;
}

int HipExec::compute_free(int s) {
  HIPCHK(c, hipEventRecord(c->slot_free[s], c->cs));
  return LSN_OK;
}

// Maps a scheduler status to the context's error (the executor's own
// failures have set the message already).
static lsn_status sched_status(lsn_ctx* c, int st) {
  if (st == 0) return LSN_OK;
  if (st == SCHED_NO_SLOT) return fail(c, LSN_ERR_STATE, "scheduler found no free slot");
  return (lsn_status)st;
}

static lsn_status layer_begin(lsn_ctx* c, int kind, int layer, const uint8_t** rec) {
  SlotScheduler<HipExec>& q = c->sched;
  if (c->pass_kind != kind) return fail(c, LSN_ERR_STATE, "layer call outside a matching pass");
  if (q.pos >= q.order.size() || q.order[q.pos] != layer)
    return fail(c, LSN_ERR_STATE, "layer %d out of order (expected %d)", layer,
                q.pos < q.order.size() ? q.order[q.pos] : -1);
  if (!c->loaded[layer]) return fail(c, LSN_ERR_STATE, "layer %d was never loaded", layer);
  if (c->cfg.mode == LSN_RESIDENT) {
    *rec = c->records + (uint64_t)layer * c->rec_bytes;
  } else {
    HipExec x{c};
    int s = -1;
    lsn_status st = sched_status(c, q.layer_begin(x, &s));
    if (st != LSN_OK) return st;
    *rec = c->records + (uint64_t)s * c->rec_bytes;
  }
  if (c->compute_delay_us) spin_us(c->compute_delay_us, c->wall_khz, c->cs);
  return LSN_OK;
}

static lsn_status layer_end(lsn_ctx* c) {
  if (c->cfg.mode == LSN_RESIDENT) {
    c->sched.pos += 1;
  } else {
    HipExec x{c};
    lsn_status st = sched_status(c, c->sched.layer_end(x));
    if (st != LSN_OK) return st;
  }
  return launch_check(c);
}

// ---------------------------------------------------------------------------
// GEMM helpers
// ---------------------------------------------------------------------------
static GemmParams base_params(const lsn_ctx* c) {
  GemmParams p;
  memcpy(p.levels, c->levels, sizeof p.levels);
  return p;
}

// projections sharing one GEMM: q|k|v, o, gate|up, down
static int group_index(Group g) {
  return g.first == LSN_Q ? 0 : g.first == LSN_O ? 1 : g.first == LSN_GATE ? 2 : 3;
}

// Forward low-rank extension of a group: t_p = x A_p (kept in lt[p]) and
// aext = bf16(s t_p) per adapted slot in one launch.  The bf16 copies it
// reads (A_p^T, and the block layout of the B_p^T for the GEMM) are cached
// per layer and rebuilt after adapter writes.
static int lora_fwd_ext(lsn_ctx* c, int layer, Group g, const uint16_t* x, int64_t ldx, int T) {
  c->fwd_bext = nullptr;
  if (!c->adapters_on) return 0;
  int nad = 0;
  for (int p = g.first; p < g.first + g.count; ++p) nad += c->targeted(p);
  if (!nad) return 0;
  const int r = c->cfg.lora_rank, kext = 16 * nad;
  LoraDown d;
  d.X = x; d.ldx = ldx; d.R = T; d.K = (int)c->K[g.first]; d.r = r;
  d.ext = c->aext; d.ld_ext = kext; d.ext_scale = c->lora_scale();
  const size_t ci = (size_t)layer * 4 + group_index(g);
  uint16_t* be = c->fext + c->fext_off[ci];
  if (c->fext_ver[ci] != c->lora_version) {  // rebuild the layer's bf16 copies
    // rows of one projection are zero in the other projections' slots
    if (g.count > 1) fill_u32(be, 0, group_rows(c, g) * kext / 2, c->cs);
    ExtBatch eb;  // bf16(B_p^T) rows and bf16(A_p)^T of every adapter, one launch
    int slot = 0;
    int64_t row0 = 0;
    for (int p = g.first; p < g.first + g.count; ++p) {
      if (c->targeted(p)) {
        eb.job[eb.n++] = ExtJob{c->B_of(layer, p), 1, c->N[p], (int)c->N[p], r,
                                be + row0 * kext, kext, 1, 16 * slot, 0};
        eb.job[eb.n++] = lora_at_job(c->A_of(layer, p), (int)c->K[p], r,
                                     c->fat + c->fat_off[(size_t)layer * NPROJ + p]);
        ++slot;
      }
      row0 += c->N[p];
    }
    (void)lora_convert(eb, c->cs);
    c->fext_ver[ci] = c->lora_version;
  }
  for (int p = g.first; p < g.first + g.count; ++p)
    if (c->targeted(p)) {
      d.AT[d.n] = c->fat + c->fat_off[(size_t)layer * NPROJ + p];
      d.t[d.n] = c->lt + (int64_t)p * T * 16;
      ++d.n;
    }
  d.part = c->lpart; d.part_floats = c->lpart_floats;
  (void)lora_down(d, c->cs);
  c->fwd_bext = be;
  return kext;
}

// Backward of the low-rank branches of a group.  dyf: fp32 gradient of the
// group's fused output [T, rows] (row stride lddy); x: forward input [T, K].
// Adds dA, dB; prepares aext = bf16(s u_p), bext = A_p (bf16) for dX.
// Three launches for all adapters of the group: u_p = dy_p B_p^T (with
// aext), dA_p += s x^T u_p (one pass over x), dB_p += s t_p^T dy_p.
static int lora_bwd_ext(lsn_ctx* c, int layer, Group g, const float* dyf, int64_t lddy,
                        const uint16_t* x, int64_t ldx, int T) {
  int nad = 0;
  for (int p = g.first; p < g.first + g.count; ++p) nad += c->targeted(p);
  if (!nad) return 0;
  const int r = c->cfg.lora_rank, kext = 16 * nad;
  const float s = c->lora_scale();
  LoraU u;
  u.dy = dyf; u.dy_f32 = 1; u.lddy = lddy; u.R = T; u.r = r;
  u.ext = c->aext; u.ld_ext = kext; u.ext_scale = s;
  LoraTGrad ga;  // dA_p += s x^T u_p, dA stored [K, r]
  ga.R = T; ga.r = r; ga.y_f32 = 0; ga.ldy = ldx; ga.scale = s; ga.njobs = 1;
  ga.job[0].Y = x; ga.job[0].C = (int)c->K[g.first]; ga.job[0].so_c = r; ga.job[0].so_j = 1;
  LoraTGrad gb;  // dB_p += s t_p^T dy_p, dB stored [r, N_p]
  gb.R = T; gb.r = r; gb.y_f32 = 1; gb.ldy = lddy; gb.scale = s;
  int64_t col0 = 0;
  for (int p = g.first; p < g.first + g.count; ++p) {
    if (c->targeted(p)) {
      const int q = u.n++;
      u.col0[q] = col0;
      u.N[q] = (int)c->N[p];
      u.B[q] = c->B_of(layer, p);
      u.u[q] = c->lu + (int64_t)q * T * 16;
      LoraTGradJob& ja = ga.job[0];
      ja.Z[ja.nz] = u.u[q];
      ja.ldz[ja.nz] = r;
      ja.out[ja.nz] = c->dA_of(layer, p);
      ++ja.nz;
      LoraTGradJob& jb = gb.job[gb.njobs++];
      jb.Y = dyf + col0;
      jb.C = (int)c->N[p];
      jb.nz = 1;
      jb.so_c = 1;
      jb.so_j = c->N[p];
      jb.Z[0] = c->lt + (int64_t)p * T * 16;
      jb.ldz[0] = r;
      jb.out[0] = c->dB_of(layer, p);
    }
    col0 += c->N[p];
  }
  if (lora_u_ok(u)) {
    (void)lora_u(u, c->lpart, c->lpart_floats, c->cs);
    // token-split partial sums in hpart (free outside the attention backward)
    const int64_t hpf = (int64_t)T * c->QD;
    (void)lora_tgrad(ga, c->hpart, hpf, c->cs);
    (void)lora_tgrad(gb, c->hpart, hpf, c->cs);
  } else {  // rows not 16-byte aligned: the general product, one adapter at a time
    for (int q = 0; q < u.n; ++q) {
      const float* dy = dyf + u.col0[q];
      LoraMM mu;  // u = dy B^T, aext = bf16(s u)
      mu.X = dy; mu.x_f32 = 1; mu.ldx = lddy; mu.R = T; mu.K = u.N[q];
      mu.W = u.B[q]; mu.sk = 1; mu.sj = u.N[q]; mu.r = r;
      mu.out = u.u[q]; mu.so_r = r; mu.so_j = 1;
      mu.ext = c->aext + 16 * q; mu.ld_ext = kext; mu.ext_scale = s;
      (void)lora_mm(mu, c->lpart, c->lpart_floats, c->cs);
      LoraMM ma;  // dA += s x^T u
      ma.X = x; ma.trans = 1; ma.ldx = ldx; ma.R = ga.job[0].C; ma.K = T;
      ma.W = u.u[q]; ma.sk = r; ma.sj = 1; ma.r = r;
      ma.out = ga.job[0].out[q]; ma.so_r = r; ma.so_j = 1; ma.accumulate = 1; ma.scale = s;
      (void)lora_mm(ma, c->lpart, c->lpart_floats, c->cs);
      LoraMM mb;  // dB += s t^T dy, stored dB[j*N + n]
      mb.X = dy; mb.x_f32 = 1; mb.trans = 1; mb.ldx = lddy; mb.R = u.N[q]; mb.K = T;
      mb.W = gb.job[q].Z[0]; mb.sk = r; mb.sj = 1; mb.r = r;
      mb.out = gb.job[q].out[0]; mb.so_r = 1; mb.so_j = u.N[q]; mb.accumulate = 1; mb.scale = s;
      (void)lora_mm(mb, c->lpart, c->lpart_floats, c->cs);
    }
  }
  ExtBatch eb;  // bext [K, kext]: bf16(A_p) of every adapter, one launch
  for (int p = g.first; p < g.first + g.count; ++p)
    if (c->targeted(p)) {
      eb.job[eb.n] = ExtJob{c->A_of(layer, p), r, 1, (int)c->K[p], r, c->bext, kext, 1, 16 * eb.n, 0};
      ++eb.n;
    }
  (void)lora_convert(eb, c->cs);
  return kext;
}

// the forward GEMM of a group: out (op)= x W_group (+ low-rank extension);
// with C_SWIGLU (gate|up only) out is a = bf16(silu(gate) * up) [T, F]
static GemmParams fwd_params(lsn_ctx* c, const uint8_t* rec, Group g, const uint16_t* x, int T,
                             int kext, void* out, int cmode, const float* res) {
  GemmParams p = base_params(c);
  const int pf = g.first;
  p.M = T;
  p.N = (int)group_rows(c, g);
  p.K = (int)c->K[pf];
  p.A = x;
  p.lda = c->K[pf];
  p.B = rec + c->code_off[pf];
  p.absmax = reinterpret_cast<const float*>(rec + c->amax_off[pf]);
  p.rowlen = c->K[pf];
  p.C = out;
  p.ldc = cmode == C_SWIGLU ? p.N / 2 : p.N;
  p.cmode = cmode;
  p.R = res;
  p.ldr = p.N;
  if (kext) {
    p.Aext = c->aext;
    p.ldae = kext;
    p.Bext = c->fwd_bext;
    p.ldbe = kext;
    p.kext = kext;
  }
  return p;
}

static hipError_t nf4_fwd_gemm(lsn_ctx* c, const uint8_t* rec, Group g, const uint16_t* x, int T,
                               int kext, void* out, int cmode, const float* res,
                               SplitSum* keep = nullptr) {
  return cgemm(c, fwd_params(c, rec, g, x, T, kext, out, cmode, res), A_BF16_K, B_NF4_K, 1, keep);
}

// dX = dY W_group (+ low-rank extension); dY is fp32 (opa A_F32_K) or bf16.
// fp32 dY is first rounded to bf16 (the value the MFMA takes anyway) into
// dqkvb, which is free from the previous layer's q|k|v input gradient until
// this layer's rope backward refills it.
static hipError_t nf4_bwd_gemm(lsn_ctx* c, const uint8_t* rec, Group g, const void* dy, int opa,
                               int T, int kext, void* out, int cmode, SplitSum* keep = nullptr) {
  GemmParams p = base_params(c);
  const int pf = g.first;
  p.M = T;
  p.N = (int)c->K[pf];
  p.K = (int)group_rows(c, g);
  if (opa == A_F32_K) {
    f32_to_bf16(static_cast<const float*>(dy), c->dqkvb, (int64_t)T * p.K, c->cs);
    dy = c->dqkvb;
    opa = A_BF16_K;
  }
  p.A = dy;
  p.lda = p.K;
  p.B = rec + c->code_off[pf];
  p.absmax = reinterpret_cast<const float*>(rec + c->amax_off[pf]);
  p.rowlen = c->K[pf];
  p.C = out;
  p.ldc = p.N;
  p.cmode = cmode;
  if (kext) {
    p.Aext = c->aext;
    p.ldae = kext;
    p.Bext = c->bext;
    p.ldbe = kext;
    p.kext = kext;
  }
  return cgemm(c, p, opa, B_NF4_R, 1, keep);
}

// ---------------------------------------------------------------------------
// one decoder layer
// ---------------------------------------------------------------------------
// final_residual: the forward of a pass (down projection and residual into
// out); otherwise the backward's recompute, which stops before down and also
// keeps the attention probabilities the backward reads
static lsn_status layer_forward(lsn_ctx* c, int layer, const uint8_t* rec, const float* h,
                                float* out, bool final_residual) {
  const lsn_config& g = c->cfg;
  const int T = c->T, S = c->seq_len, H = g.hidden, F = g.ffn, d = g.head_dim;
  const int nq = g.n_heads, nkv = g.n_kv_heads, grp = nq / nkv;
  const int QKV = c->QKV, QD = c->QD, KVD = c->KVD;
  const uint16_t* g1 = reinterpret_cast<const uint16_t*>(rec + c->norm_off[0]);
  const uint16_t* g2 = reinterpret_cast<const uint16_t*>(rec + c->norm_off[1]);
  hipStream_t s = c->cs;

  rmsnorm_fwd(h, g1, T, H, g.rms_eps, c->n1, c->rstd1, s);
  int kext = lora_fwd_ext(c, layer, G_QKV, c->n1, H, T);
  // split-k partial sums of the projections go straight to their consumers
  // (rope, the residual RMSNorm, the SwiGLU and RMSNorm backwards), which add
  // them as the reduction would
  SplitSum ss;
  const bool rope_f = rope_fwd_fuses(d, c->qkvb);
  HIPCHK(c, nf4_fwd_gemm(c, rec, G_QKV, c->n1, T, kext, c->qkv, C_F32, nullptr,
                         rope_f ? &ss : nullptr));
  if (rope_f) rope_fwd(ss, c->qkvb, T, S, nq, nkv, d, g.rope_theta, s);
  else rope_fwd(c->qkv, c->qkvb, T, S, nq, nkv, d, g.rope_theta, s);

  // attention: one fused kernel where the shape allows (S <= 512, d 64 or
  // 128), else scores, softmax and P v as three launches
  // fragment-ordered operands in dqkv, free until the backward's attention
  uint16_t* frag = reinterpret_cast<uint16_t*>(c->dqkv);
  if (attn_fwd_ok(S, d, QKV, QD, c->qkvb, c->O, frag)) {
    AttnFwdParams ap;
    ap.qkv = c->qkvb; ap.ld = QKV; ap.frag = frag;
    ap.O = c->O; ap.ldo = QD;
    ap.Pf = final_residual ? nullptr : c->Pf;
    ap.Pb = final_residual ? nullptr : c->Pb;
    ap.n_seq = c->n_seq; ap.S = S; ap.nq = nq; ap.nkv = nkv;
    ap.alpha = 1.0f / sqrtf((float)d);
    HIPCHK(c, attn_fwd(ap, d, s));
  } else {
    // attention: scores = q k^T / sqrt(d) per (sequence, head)
    {
      GemmParams p = base_params(c);
      p.M = S; p.N = S; p.K = d;
      p.A = c->qkvb; p.lda = QKV;
      p.B = c->qkvb + QD; p.ldb = QKV;
      p.zdiv = nq; p.grpB = grp;
      p.sA_o = (int64_t)S * QKV; p.sA_i = d;
      p.sB_o = (int64_t)S * QKV; p.sB_i = d;
      p.C = c->scores; p.ldc = S;
      p.sC_o = (int64_t)nq * S * S; p.sC_i = (int64_t)S * S;
      p.alpha = 1.0f / sqrtf((float)d);
      p.causal = CAUSAL_SKIP_UPPER;  // the softmax reads keys <= query only
      HIPCHK(c, cgemm(c, p, A_BF16_K, B_BF16_K, c->n_seq * nq));
    }
    softmax_causal(c->scores, c->Pf, c->Pb, S, (int64_t)c->n_seq * nq * S, s);
    {  // O = P V
      GemmParams p = base_params(c);
      p.M = S; p.N = d; p.K = S;
      p.A = c->Pb; p.lda = S;
      p.B = c->qkvb + QD + KVD; p.ldb = QKV;
      p.zdiv = nq; p.grpB = grp;
      p.sA_o = (int64_t)nq * S * S; p.sA_i = (int64_t)S * S;
      p.sB_o = (int64_t)S * QKV; p.sB_i = d;
      p.C = c->O; p.ldc = QD; p.cmode = C_BF16;
      p.sC_o = (int64_t)S * QD; p.sC_i = d;
      p.causal = CAUSAL_K_TO_ROW;  // P is zero for keys > query
      HIPCHK(c, cgemm(c, p, A_BF16_K, B_BF16_R, c->n_seq * nq));
    }
  }
  kext = lora_fwd_ext(c, layer, G_O, c->O, QD, T);
  if (rmsnorm_fwd_res_fuses(H, h, c->h2, g2, c->n2)) {  // h2 = h + o(...), then its norm
    HIPCHK(c, nf4_fwd_gemm(c, rec, G_O, c->O, T, kext, c->h2, C_F32_RES, h, &ss));
    if (ss.ns > 1) rmsnorm_fwd_res(h, ss, g2, T, H, g.rms_eps, c->h2, c->n2, c->rstd2, s);
    else rmsnorm_fwd(c->h2, g2, T, H, g.rms_eps, c->n2, c->rstd2, s);
  } else {
    HIPCHK(c, nf4_fwd_gemm(c, rec, G_O, c->O, T, kext, c->h2, C_F32_RES, h));
    rmsnorm_fwd(c->h2, g2, T, H, g.rms_eps, c->n2, c->rstd2, s);
  }
  kext = lora_fwd_ext(c, layer, G_GU, c->n2, H, T);
  // The forward writes a = silu(gate) * up straight from the gate|up GEMM's
  // accumulators where its kernel allows; the backward's recompute keeps
  // gate and up (fp32) for the SwiGLU backward and rebuilds a from them only
  // when the down adapter's gradients need it.  Both launches use the same
  // tile plan, so a is the same either way.
  const GemmParams pgu = fwd_params(c, rec, G_GU, c->n2, T, kext, c->a, C_SWIGLU, nullptr);
  if (final_residual && nf4f_swiglu_ok(pgu)) {
    HIPCHK(c, cgemm(c, pgu, A_BF16_K, B_NF4_K, 1));
  } else {
    HIPCHK(c, nf4_fwd_gemm(c, rec, G_GU, c->n2, T, kext, c->gu, C_F32, nullptr));
    if (final_residual || (c->adapters_on && c->targeted(LSN_DOWN))) swiglu_fwd(c->gu, c->a, T, F, s);
  }
  kext = lora_fwd_ext(c, layer, G_D, c->a, F, T);  // also keeps t of down for backward
  if (final_residual)
    HIPCHK(c, nf4_fwd_gemm(c, rec, G_D, c->a, T, kext, out, C_F32_RES, c->h2));
  return launch_check(c);
}

static lsn_status layer_backward(lsn_ctx* c, int layer, const uint8_t* rec, const float* h,
                                 const float* dout, float* dh) {
  const lsn_config& g = c->cfg;
  const int T = c->T, S = c->seq_len, H = g.hidden, F = g.ffn, d = g.head_dim;
  const int nq = g.n_heads, nkv = g.n_kv_heads, grp = nq / nkv;
  const int QKV = c->QKV, QD = c->QD, KVD = c->KVD;
  const uint16_t* g1 = reinterpret_cast<const uint16_t*>(rec + c->norm_off[0]);
  const uint16_t* g2 = reinterpret_cast<const uint16_t*>(rec + c->norm_off[1]);
  hipStream_t s = c->cs;

  // recompute the forward activations of this layer (adapters on)
  lsn_status st = layer_forward(c, layer, rec, h, nullptr, false);
  if (st != LSN_OK) return st;

  // MLP: out = h2 + down(silu(gate) * up)
  int kext = lora_bwd_ext(c, layer, G_D, dout, H, c->a, F, T);
  const bool gu_ad = c->targeted(LSN_GATE) || c->targeted(LSN_UP);
  SplitSum ss;
  const bool sw_f = swiglu_bwd_fuses(T, F, c->gu, c->dgu, gu_ad ? c->dguf : nullptr);
  HIPCHK(c, nf4_bwd_gemm(c, rec, G_D, dout, A_F32_K, T, kext, c->da, C_F32, sw_f ? &ss : nullptr));
  if (sw_f) swiglu_bwd(c->gu, ss, c->dgu, gu_ad ? c->dguf : nullptr, T, F, s);
  else swiglu_bwd(c->gu, c->da, c->dgu, gu_ad ? c->dguf : nullptr, T, F, s);
  kext = lora_bwd_ext(c, layer, G_GU, c->dguf, 2 * F, c->n2, H, T);
  const bool n2_f = rmsnorm_bwd_fuses(H, c->h2, c->dh2, dout, g2);
  HIPCHK(c, nf4_bwd_gemm(c, rec, G_GU, c->dgu, A_BF16_K, T, kext, c->dn, C_F32, n2_f ? &ss : nullptr));
  // dh2 also in bf16 (dqkvb, free until the rope backward), the o input
  // gradient GEMM's operand
  if (n2_f) rmsnorm_bwd(c->h2, g2, c->rstd2, ss, dout, T, H, c->dh2, c->dqkvb, s);
  else rmsnorm_bwd(c->h2, g2, c->rstd2, SplitSum{c->dn, 1, 0}, dout, T, H, c->dh2, c->dqkvb, s);

  // attention block: h2 = h + o(attn(rope(q), rope(k), v))
  kext = lora_bwd_ext(c, layer, G_O, c->dh2, H, c->O, QD, T);
  HIPCHK(c, nf4_bwd_gemm(c, rec, G_O, c->dqkvb, A_BF16_K, T, kext, c->dO, C_BF16));
  const int Z = c->n_seq * nq;
  const float scale = 1.0f / sqrtf((float)d);
  // dP, dS and dQ in one fused kernel where the shape allows (its operand
  // copies go to qkv, free after the recompute's rope); it overwrites Pb
  // with dS, so dV (from P) runs first
  uint16_t* bfrag = reinterpret_cast<uint16_t*>(c->qkv);
  const bool fused = attn_bwd_ok(S, d, QKV, QD, QKV, c->qkvb, c->dO, c->dqkv, bfrag, c->Pf);
  if (!fused) {
    {  // dP = dO V^T
      GemmParams p = base_params(c);
      p.M = S; p.N = S; p.K = d;
      p.A = c->dO; p.lda = QD;
      p.B = c->qkvb + QD + KVD; p.ldb = QKV;
      p.zdiv = nq; p.grpB = grp;
      p.sA_o = (int64_t)S * QD; p.sA_i = d;
      p.sB_o = (int64_t)S * QKV; p.sB_i = d;
      p.C = c->scores; p.ldc = S;
      p.sC_o = (int64_t)nq * S * S; p.sC_i = (int64_t)S * S;
      p.causal = CAUSAL_SKIP_UPPER;  // the softmax backward reads keys <= query only
      HIPCHK(c, cgemm(c, p, A_BF16_K, B_BF16_K, Z));
    }
  }
  // dV[kv] = sum over its q heads of P_h^T dO_h: one product per q head
  // (batch n_seq x nq, 4x the workgroups of a product per kv head), then
  // the group sums in head order
  {
    GemmParams p = base_params(c);
    p.M = S; p.N = d; p.K = S;
    p.A = c->Pb; p.lda = S;
    p.B = c->dO; p.ldb = QD;
    p.zdiv = nq; p.grpB = 1;
    p.sA_o = (int64_t)nq * S * S; p.sA_i = (int64_t)S * S;
    p.sB_o = (int64_t)S * QD; p.sB_i = d;
    p.C = c->hpart; p.ldc = d;
    p.sC_o = (int64_t)nq * S * d; p.sC_i = (int64_t)S * d;
    p.causal = CAUSAL_K_FROM_ROW;  // P^T is zero for queries < key
    HIPCHK(c, cgemm(c, p, A_BF16_R, B_BF16_R, Z));
    group_sum(c->hpart, c->n_seq, nq, grp, S, d, c->dqkv + QD + KVD, QKV, s);
  }
  if (fused) {
    AttnBwdParams ab;
    ab.qkv = c->qkvb; ab.ld = QKV; ab.dO = c->dO; ab.lddo = QD; ab.frag = bfrag;
    ab.Pin = c->Pf; ab.dS = c->Pb; ab.dQ = c->dqkv; ab.ldq = QKV;
    ab.n_seq = c->n_seq; ab.S = S; ab.nq = nq; ab.nkv = nkv; ab.alpha = scale;
    HIPCHK(c, attn_bwd(ab, d, s));
  } else {
    softmax_bwd(c->Pf, c->scores, c->Pb, S, (int64_t)Z * S, s);  // dS (bf16) over Pb
    {  // dQ = scale dS K
      GemmParams p = base_params(c);
      p.M = S; p.N = d; p.K = S;
      p.A = c->Pb; p.lda = S;
      p.B = c->qkvb + QD; p.ldb = QKV;
      p.zdiv = nq; p.grpB = grp;
      p.sA_o = (int64_t)nq * S * S; p.sA_i = (int64_t)S * S;
      p.sB_o = (int64_t)S * QKV; p.sB_i = d;
      p.C = c->dqkv; p.ldc = QKV;
      p.sC_o = (int64_t)S * QKV; p.sC_i = d;
      p.alpha = scale;
      p.causal = CAUSAL_K_TO_ROW;  // dS is zero for keys > query
      HIPCHK(c, cgemm(c, p, A_BF16_K, B_BF16_R, Z));
    }
  }
  {  // dK[kv] = scale sum over its q heads of dS_h^T Q_h, as dV
    GemmParams p = base_params(c);
    p.M = S; p.N = d; p.K = S;
    p.A = c->Pb; p.lda = S;
    p.B = c->qkvb; p.ldb = QKV;
    p.zdiv = nq; p.grpB = 1;
    p.sA_o = (int64_t)nq * S * S; p.sA_i = (int64_t)S * S;
    p.sB_o = (int64_t)S * QKV; p.sB_i = d;
    p.C = c->hpart; p.ldc = d;
    p.sC_o = (int64_t)nq * S * d; p.sC_i = (int64_t)S * d;
    p.alpha = scale;
    p.causal = CAUSAL_K_FROM_ROW;  // dS^T is zero for queries < key
    HIPCHK(c, cgemm(c, p, A_BF16_R, B_BF16_R, Z));
    group_sum(c->hpart, c->n_seq, nq, grp, S, d, c->dqkv + QD, QKV, s);
  }
  rope_bwd(c->dqkv, c->dqkvb, T, S, nq, nkv, d, g.rope_theta, s);
  kext = lora_bwd_ext(c, layer, G_QKV, c->dqkv, QKV, c->n1, H, T);
  const bool n1_f = rmsnorm_bwd_fuses(H, h, dh, c->dh2, g1);
  HIPCHK(c, nf4_bwd_gemm(c, rec, G_QKV, c->dqkvb, A_BF16_K, T, kext, c->dn, C_F32, n1_f ? &ss : nullptr));
  if (n1_f) rmsnorm_bwd(h, g1, c->rstd1, ss, c->dh2, T, H, dh, nullptr, s);
  else rmsnorm_bwd(h, g1, c->rstd1, c->dn, c->dh2, T, H, dh, s);
  return launch_check(c);
}

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

lsn_status lsn_nf4_codebook(float* out16) {
  if (!out16) return LSN_ERR_INVALID;
  nf4_levels(out16);
  return LSN_OK;
}

lsn_status lsn_nf4_quantize(const float* w, uint64_t n, uint8_t* codes, float* absmax) {
  if (!w || !codes || !absmax) return n == 0 ? LSN_OK : LSN_ERR_INVALID;
  return nf4_quantize(w, n, codes, absmax) ? LSN_OK : LSN_ERR_INVALID;
}

lsn_status lsn_nf4_dequantize(const uint8_t* codes, const float* absmax, uint64_t n,
                                   float* w) {
  if (!codes || !absmax || !w) return n == 0 ? LSN_OK : LSN_ERR_INVALID;
  nf4_dequantize_host(codes, absmax, n, w);
  return LSN_OK;
}

lsn_status lsn_nf4_dequant(const uint8_t* codes, const float* absmax, uint64_t n, void* out,
                           int32_t out_bf16, void* hip_stream) {
  if (n == 0) return LSN_OK;
  if (!codes || !absmax || !out || n % 8) return LSN_ERR_INVALID;
  (void)hipGetLastError();  // a status left by the caller's HIP calls is not ours
  float lv[16];
  nf4_levels(lv);
  nf4_dequant(codes, absmax, (int64_t)n, lv, out_bf16 ? nullptr : (float*)out,
              out_bf16 ? (uint16_t*)out : nullptr, (hipStream_t)hip_stream);
  return launch_status0("lsn_nf4_dequant");
}

// Scratch of the stateless projection: t, u fp32 [M,16]; aext bf16 [M,16];
// bext bf16 [max(N,K),16]; split-k partial sums of the low-rank products and
// of the GEMM.
struct LinScratch {
  float *t = nullptr, *u = nullptr, *lpart = nullptr, *gpart = nullptr;
  uint16_t *aext = nullptr, *bext = nullptr;
  int64_t lpf = 0, gpf = 0;
  uint64_t bytes = 0;
};

static LinScratch lin_scratch(char* base, int M, int K, int N) {
  LinScratch L;
  Carver cv;
  auto P = [&](uint64_t b) -> char* { const uint64_t o = cv.take(b); return base ? base + o : nullptr; };
  L.lpf = std::max<int64_t>({lora_mm_partial_floats(M, K), lora_mm_partial_floats(M, N),
                             lora_mm_partial_floats(K, M), lora_mm_partial_floats(N, M),
                             lora_down_partial_floats(M, K, 1)});
  L.gpf = std::max(gemm_partial_floats(M, N, K, 1, 1), gemm_partial_floats(M, K, N, 1, 1));
  L.t = (float*)P((uint64_t)M * 16 * 4);
  L.u = (float*)P((uint64_t)M * 16 * 4);
  L.aext = (uint16_t*)P((uint64_t)M * 16 * 2);
  L.bext = (uint16_t*)P((uint64_t)std::max(N, K) * 16 * 2);
  L.lpart = (float*)P((uint64_t)L.lpf * 4);
  L.gpart = (float*)P((uint64_t)L.gpf * 4);
  L.bytes = align_up(cv.off, 256);
  return L;
}

lsn_status lsn_nf4_linear_scratch_bytes(int32_t M, int32_t K, int32_t N, int32_t r,
                                        uint64_t* bytes) {
  if (!bytes || M < 0 || K <= 0 || N <= 0 || r < 0 || r > 16) return LSN_ERR_INVALID;
  *bytes = lin_scratch(nullptr, M, K, N).bytes;
  return LSN_OK;
}

static lsn_status linear_args_ok(const uint8_t* codes, const float* absmax, int32_t M, int32_t K,
                                 int32_t N, const void* X, const float* A, const float* B,
                                 int32_t r, void* scratch, uint64_t sb) {
  if (!codes || !absmax || !X || M < 0 || K <= 0 || N <= 0) return LSN_ERR_INVALID;
  if (K % 16 || N % 8) return LSN_ERR_INVALID;
  if (r < 0 || r > 16) return LSN_ERR_INVALID;
  if (r > 0 && (!A || !B)) return LSN_ERR_INVALID;
  if (r > 0 && (!scratch || sb < lin_scratch(nullptr, M, K, N).bytes)) return LSN_ERR_INVALID;
  return LSN_OK;
}

// Without enough scratch (allowed when r = 0) the GEMM runs without split-k.
static LinScratch lin_scratch_or_none(void* scratch, uint64_t sb, int M, int K, int N) {
  LinScratch L = lin_scratch(nullptr, M, K, N);
  if (!scratch || sb < L.bytes) return LinScratch();
  return lin_scratch((char*)scratch, M, K, N);
}

// The forward projection on carved scratch L (adapter products, then the
// NF4 GEMM with the low-rank extension; split-k partial sums in L.gpart).
static lsn_status linear_fwd_core(const uint8_t* codes, const float* absmax, int32_t M, int32_t K,
                                  int32_t N, const uint16_t* X, const float* A, const float* B,
                                  int32_t r, float s, float* Y, const LinScratch& L,
                                  hipStream_t hs, const char* what) {
  GemmParams p;
  nf4_levels(p.levels);
  p.M = M; p.N = N; p.K = K;
  p.A = X; p.lda = K;
  p.B = codes; p.absmax = absmax; p.rowlen = K;
  p.C = Y; p.ldc = N;
  p.part = L.gpart; p.part_floats = L.gpf;
  if (r > 0) {
    // t = X A and aext = bf16(s t) from the fp32 A (split over k, then the
    // ordered sum), and bext = bf16(B^T) [N, 16] from the fp32 B in the same
    // launches
    LoraDown d;
    d.X = X; d.ldx = K; d.R = M; d.K = K; d.r = r; d.n = 1;
    d.AF[0] = A; d.t[0] = L.t;
    d.ext = L.aext; d.ld_ext = 16; d.ext_scale = s;
    d.conv.W = B; d.conv.srow = 1; d.conv.sj = N; d.conv.rows = N; d.conv.r = r;
    d.conv.out = L.bext; d.conv.ld = 16; d.conv.c0 = 0;
    d.part = L.lpart; d.part_floats = L.lpf;
    (void)lora_down(d, hs);
    p.Aext = L.aext; p.ldae = 16; p.Bext = L.bext; p.ldbe = 16; p.kext = 16;
  }
  const hipError_t e = gemm(p, A_BF16_K, B_NF4_K, 1, hs);
  if (e != hipSuccess) return fail0(LSN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return launch_status0(what);
}

lsn_status lsn_nf4_linear_fwd(const uint8_t* codes, const float* absmax, int32_t M, int32_t K,
                              int32_t N, const uint16_t* X, const float* A, const float* B,
                              int32_t r, float s, float* Y, void* scratch, uint64_t sb,
                              void* hip_stream) {
  lsn_status st = linear_args_ok(codes, absmax, M, K, N, X, A, B, r, scratch, sb);
  if (st != LSN_OK || !Y) return st != LSN_OK ? st : LSN_ERR_INVALID;
  if (M == 0) return LSN_OK;
  (void)hipGetLastError();  // a status left by the caller's HIP calls is not ours
  const LinScratch L = lin_scratch_or_none(scratch, sb, M, K, N);
  return linear_fwd_core(codes, absmax, M, K, N, X, A, B, r, s, Y, L, (hipStream_t)hip_stream,
                         "lsn_nf4_linear_fwd");
}

// ---------------------------------------------------------------------------
// The same forward projection for callers that cannot allocate: its scratch
// is this file-scope device array.  Host code never uses the array's name as
// an address (on the host it names a stand-in, not device memory): each
// device's address comes from hipGetSymbolAddress, taken once per device on
// the first call there with that device current, and only that address is
// passed to kernels.
// ---------------------------------------------------------------------------
constexpr uint64_t NOALLOC_SCRATCH_BYTES = 64ull << 20;
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};
}  // namespace

// The forward's share of the stateless scratch: t, aext [M, 16], bext
// [N, 16], the down-projection's and the NF4 GEMM's split-k partials of this
// shape only (the same splits the scratch-taking call uses).
static LinScratch lin_scratch_fwd(char* base, int M, int K, int N) {
  LinScratch L;
  Carver cv;
  auto P = [&](uint64_t b) -> char* { const uint64_t o = cv.take(b); return base ? base + o : nullptr; };
  L.lpf = lora_down_partial_floats(M, K, 1);
  L.gpf = gemm_partial_floats(M, N, K, 1, 1);
  L.t = (float*)P((uint64_t)M * 16 * 4);
  L.aext = (uint16_t*)P((uint64_t)M * 16 * 2);
  L.bext = (uint16_t*)P((uint64_t)N * 16 * 2);
  L.lpart = (float*)P((uint64_t)std::max<int64_t>(L.lpf, 1) * 4);
  L.gpart = (float*)P((uint64_t)std::max<int64_t>(L.gpf, 1) * 4);
  L.bytes = align_up(cv.off, 256);
  return L;
}

lsn_status lsn_nf4_linear_fwd_noalloc(const uint8_t* codes, const float* absmax, int32_t M,
                                      int32_t K, int32_t N, const uint16_t* X, const float* A,
                                      const float* B, int32_t r, float s, float* Y,
                                      void* hip_stream) {
  if (!codes || !absmax || !X || !Y || M < 0 || K <= 0 || N <= 0 || K % 16 || N % 8 || r < 0 ||
      r > 16 || (r > 0 && (!A || !B)))
    return fail0(LSN_ERR_INVALID, "lsn_nf4_linear_fwd_noalloc: bad arguments");
  const uint64_t need = lin_scratch_fwd(nullptr, M, K, N).bytes;
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail0(LSN_ERR_INVALID,
                 "lsn_nf4_linear_fwd_noalloc: %d x %d -> %d needs %llu bytes of scratch, more "
                 "than the %llu of the fixed device array",
                 M, K, N, (unsigned long long)need, (unsigned long long)NOALLOC_SCRATCH_BYTES);
  if (M == 0) return LSN_OK;
  (void)hipGetLastError();  // a status left by the caller's HIP calls is not ours
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES)
    return fail0(LSN_ERR_HIP, "lsn_nf4_linear_fwd_noalloc: no usable current device");
  char* base;
  {
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* ptr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !ptr)
        return fail0(LSN_ERR_HIP, "lsn_nf4_linear_fwd_noalloc: scratch address: %s",
                     hipGetErrorString(e));
      g_scratch_ptr[dev] = (char*)ptr;
    }
    base = g_scratch_ptr[dev];
  }
  const LinScratch L = lin_scratch_fwd(base, M, K, N);
  return linear_fwd_core(codes, absmax, M, K, N, X, A, B, r, s, Y, L, (hipStream_t)hip_stream,
                         "lsn_nf4_linear_fwd_noalloc");
}

lsn_status lsn_nf4_linear_bwd(const uint8_t* codes, const float* absmax, int32_t M, int32_t K,
                              int32_t N, const uint16_t* X, const float* A, const float* B,
                              int32_t r, float s, const uint16_t* dY, float* dX, float* dA,
                              float* dB, void* scratch, uint64_t sb, void* hip_stream) {
  lsn_status st = linear_args_ok(codes, absmax, M, K, N, X, A, B, r, scratch, sb);
  if (st != LSN_OK) return st;
  if (!dY || !dX || (r > 0 && (!dA || !dB))) return LSN_ERR_INVALID;
  (void)hipGetLastError();  // a status left by the caller's HIP calls is not ours
  hipStream_t hs = (hipStream_t)hip_stream;
  if (M == 0) {  // no tokens: zero adapter gradients
    if (r > 0) {
      fill_u32(dA, 0, (int64_t)K * r, hs);
      fill_u32(dB, 0, (int64_t)r * N, hs);
    }
    return launch_status0("lsn_nf4_linear_bwd");
  }
  const LinScratch L = lin_scratch_or_none(scratch, sb, M, K, N);
  GemmParams p;
  nf4_levels(p.levels);
  p.M = M; p.N = K; p.K = N;
  p.A = dY; p.lda = N;
  p.B = codes; p.absmax = absmax; p.rowlen = K;
  p.C = dX; p.ldc = K;
  p.part = L.gpart; p.part_floats = L.gpf;
  if (r > 0) {
    // t = X A (the forward's bits) and bext = bf16(A) [K, 16] from the fp32
    // A, in the same launches
    LoraDown d;
    d.X = X; d.ldx = K; d.R = M; d.K = K; d.r = r; d.n = 1;
    d.AF[0] = A; d.t[0] = L.t;
    d.conv.W = A; d.conv.srow = r; d.conv.sj = 1; d.conv.rows = K; d.conv.r = r;
    d.conv.out = L.bext; d.conv.ld = 16; d.conv.c0 = 0;
    d.part = L.lpart; d.part_floats = L.lpf;
    (void)lora_down(d, hs);
    LoraU uu;  // u = dY B^T, aext = bf16(s u)
    uu.dy = dY; uu.dy_f32 = 0; uu.lddy = N; uu.R = M; uu.r = r; uu.n = 1;
    uu.N[0] = N; uu.B[0] = B; uu.u[0] = L.u;
    uu.ext = L.aext; uu.ld_ext = 16; uu.ext_scale = s;
    if (lora_u_ok(uu)) {
      (void)lora_u(uu, L.lpart, L.lpf, hs);
    } else {
      LoraMM mu;
      mu.X = dY; mu.ldx = N; mu.R = M; mu.K = N;
      mu.W = B; mu.sk = 1; mu.sj = N; mu.r = r;
      mu.out = L.u; mu.so_r = r; mu.so_j = 1;
      mu.ext = L.aext; mu.ld_ext = 16; mu.ext_scale = s;
      (void)lora_mm(mu, L.lpart, L.lpf, hs);
    }
    LoraTGrad ga;  // dA = s X^T u (every element written: no accumulation)
    ga.R = M; ga.r = r; ga.y_f32 = 0; ga.ldy = K; ga.scale = s; ga.njobs = 1; ga.accumulate = 0;
    ga.job[0].Y = X; ga.job[0].C = K; ga.job[0].nz = 1; ga.job[0].so_c = r; ga.job[0].so_j = 1;
    ga.job[0].Z[0] = L.u; ga.job[0].ldz[0] = r; ga.job[0].out[0] = dA;
    (void)lora_tgrad(ga, L.lpart, L.lpf, hs);
    LoraTGrad gb;  // dB = s t^T dY, stored dB[j*N + n]
    gb.R = M; gb.r = r; gb.y_f32 = 0; gb.ldy = N; gb.scale = s; gb.njobs = 1; gb.accumulate = 0;
    gb.job[0].Y = dY; gb.job[0].C = N; gb.job[0].nz = 1; gb.job[0].so_c = 1; gb.job[0].so_j = N;
    gb.job[0].Z[0] = L.t; gb.job[0].ldz[0] = r; gb.job[0].out[0] = dB;
    (void)lora_tgrad(gb, L.lpart, L.lpf, hs);
    p.Aext = L.aext; p.ldae = 16; p.Bext = L.bext; p.ldbe = 16; p.kext = 16;
  }
  const hipError_t e = gemm(p, A_BF16_K, B_NF4_R, 1, hs);
  if (e != hipSuccess) return fail0(LSN_ERR_HIP, "lsn_nf4_linear_bwd: %s", hipGetErrorString(e));
  return launch_status0("lsn_nf4_linear_bwd");
}

lsn_status lsn_workspace_bytes(const lsn_config* cfg, uint64_t* bytes) {
  std::string why;
  if (!bytes) return LSN_ERR_INVALID;
  if (!cfg_valid(cfg, &why)) return fail0(LSN_ERR_INVALID, "lsn_workspace_bytes: %s", why.c_str());
  lsn_ctx tmp;
  tmp.cfg = *cfg;
  record_layout(&tmp);
  if (!layout_valid(&tmp, &why))
    return fail0(LSN_ERR_INVALID, "lsn_workspace_bytes: %s", why.c_str());
  *bytes = carve(&tmp, nullptr);
  return LSN_OK;
}

lsn_status lsn_config_record_bytes(const lsn_config* cfg, uint64_t* bytes) {
  std::string why;
  if (!bytes) return LSN_ERR_INVALID;
  if (!cfg_valid(cfg, &why)) return fail0(LSN_ERR_INVALID, "lsn_config_record_bytes: %s", why.c_str());
  lsn_ctx tmp;
  tmp.cfg = *cfg;
  record_layout(&tmp);
  *bytes = tmp.rec_bytes;
  return LSN_OK;
}

lsn_status lsn_create(const lsn_config* cfg, void* dev_ws, uint64_t ws_bytes, void* hip_stream,
                      lsn_ctx** out) {
  std::string why;
  if (!out) return LSN_ERR_INVALID;
  *out = nullptr;
  if (!cfg_valid(cfg, &why)) return fail0(LSN_ERR_INVALID, "lsn_create: %s", why.c_str());
  (void)hipGetLastError();  // a status left by the caller's HIP calls is not ours
  lsn_ctx* c = new lsn_ctx();
  c->cfg = *cfg;
  c->nslots = slot_count(cfg);
  c->sched.init(c->nslots);
  if (cfg->store_path) c->store_path = cfg->store_path;
  c->cfg.store_path = c->store_path.c_str();
  record_layout(c);
  if (!layout_valid(c, &why)) {
    delete c;
    return fail0(LSN_ERR_INVALID, "lsn_create: %s", why.c_str());
  }
  c->ws_needed = carve(c, nullptr);
  if (!dev_ws || ws_bytes < c->ws_needed || (cfg->vram_budget && c->ws_needed > cfg->vram_budget)) {
    const unsigned long long need = c->ws_needed;
    delete c;
    return fail0(LSN_ERR_NOFIT, "lsn_create: the workspace needs %llu bytes", need);
  }
  c->ws = (char*)dev_ws;
  c->ws_bytes = ws_bytes;
  carve(c, c->ws);
  c->cs = (hipStream_t)hip_stream;
  nf4_levels(c->levels);
  c->loaded.assign(cfg->n_layers, 0);
  auto cleanup = [&](lsn_status st) {
    const int en = errno;
    const hipError_t e = hipGetLastError();
    fail0(st, "lsn_create: %s", st == LSN_ERR_IO ? strerror(en) : hipGetErrorString(e));
    lsn_destroy(c);
    return st;
  };
  if (hipGetDevice(&c->device) != hipSuccess) return cleanup(LSN_ERR_HIP);
  if (hipStreamCreateWithFlags(&c->copy, hipStreamNonBlocking) != hipSuccess)
    return cleanup(LSN_ERR_HIP);
  for (int i = 0; i < c->nslots; ++i)
    if (hipEventCreateWithFlags(&c->copy_done[i], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->slot_free[i], hipEventDisableTiming) != hipSuccess)
      return cleanup(LSN_ERR_HIP);
  if (hipDeviceGetAttribute(&c->wall_khz, hipDeviceAttributeWallClockRate, c->device) != hipSuccess ||
      c->wall_khz <= 0)
    return cleanup(LSN_ERR_HIP);
  if (cfg->mode == LSN_STREAM_FILE) {
    c->fd = open(c->store_path.c_str(), O_RDWR | O_CREAT, 0644);
    if (c->fd < 0) return cleanup(LSN_ERR_IO);
    // Record reads bypass the page cache, so a step reads the device and a
    // store larger than host memory streams without evicting everything
    // else.  Records are 4 KiB multiples at 4 KiB offsets and the bounce
    // buffers are page aligned, as O_DIRECT asks.  A file system without
    // O_DIRECT (tmpfs) falls back to buffered reads.
    c->dfd = open(c->store_path.c_str(), O_RDONLY | O_DIRECT);
    for (int i = 0; i < 2; ++i) {
      void* m = mmap(nullptr, c->rec_bytes, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS, -1, 0);
      if (m == MAP_FAILED) return cleanup(LSN_ERR_IO);
      c->rd.buf[i] = (uint8_t*)m;
    }
    c->rd.th = std::thread(reader_main, c);
    for (int i = 0; i < c->nslots; ++i)
      if (hipHostMalloc((void**)&c->bounce[i], c->rec_bytes, hipHostMallocDefault) != hipSuccess)
        return cleanup(LSN_ERR_HIP);
  } else {
    if (hipHostMalloc((void**)&c->store, (uint64_t)cfg->n_layers * c->rec_bytes,
                      hipHostMallocDefault) != hipSuccess)
      return cleanup(LSN_ERR_HIP);
  }
  // adapters start at zero (A and B); gradients at zero
  fill_u32(c->lora_p, 0, (int64_t)c->lora_n, c->cs);
  fill_u32(c->lora_g, 0, (int64_t)c->lora_n, c->cs);
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(c->cs) != hipSuccess)
    return cleanup(LSN_ERR_HIP);
  *out = c;
  return LSN_OK;
}

void lsn_destroy(lsn_ctx* c) {
  if (!c) return;
  // teardown: errors here have nowhere to go
  if (c->copy) (void)hipStreamSynchronize(c->copy);
  (void)hipStreamSynchronize(c->cs);
  for (int i = 0; i < MAX_SLOTS; ++i) {
    if (c->copy_done[i]) (void)hipEventDestroy(c->copy_done[i]);
    if (c->slot_free[i]) (void)hipEventDestroy(c->slot_free[i]);
    if (c->bounce[i]) (void)hipHostFree(c->bounce[i]);
  }
  for (hipEvent_t e : c->evpool) (void)hipEventDestroy(e);
  if (c->lm_head_h && c->lm_head_h != c->embed_h) (void)hipHostFree(c->lm_head_h);
  if (c->embed_h) (void)hipHostFree(c->embed_h);
  if (c->copy) (void)hipStreamDestroy(c->copy);
  if (c->store) (void)hipHostFree(c->store);
  if (c->rd.th.joinable()) {
    {
      std::lock_guard<std::mutex> g(c->rd.mu);
      c->rd.quit = true;
    }
    c->rd.cv.notify_all();
    c->rd.th.join();
  }
  for (uint8_t* b : c->rd.buf)
    if (b) munmap(b, c->rec_bytes);
  if (c->dfd >= 0) close(c->dfd);
  if (c->fd >= 0) close(c->fd);
  delete c;
}

const char* lsn_last_error(const lsn_ctx* c) {
  if (c) return c->err.c_str();
  return g_err.empty() ? "no error recorded by a call without a context" : g_err.c_str();
}

lsn_status lsn_sync(lsn_ctx* c) {
  CHECK_CTX(c);
  HIPCHK(c, hipStreamSynchronize(c->copy));
  HIPCHK(c, hipStreamSynchronize(c->cs));
  HIPCHK(c, hipGetLastError());
  return LSN_OK;
}

lsn_status lsn_record_bytes(const lsn_ctx* c, uint64_t* bytes) {
  if (!c || !bytes) return LSN_ERR_INVALID;
  *bytes = c->rec_bytes;
  return LSN_OK;
}

lsn_status lsn_file_direct_io(const lsn_ctx* c, int32_t* direct) {
  if (!c || !direct) return LSN_ERR_INVALID;
  *direct = c->dfd >= 0 ? 1 : 0;
  return LSN_OK;
}

lsn_status lsn_load_layer_nf4(lsn_ctx* c, int32_t layer, const uint8_t* const* codes,
                              const float* const* absmax, const uint16_t* attn_norm,
                              const uint16_t* mlp_norm) {
  CHECK_CTX(c);
  if (layer < 0 || layer >= c->cfg.n_layers || !codes || !absmax || !attn_norm || !mlp_norm)
    return fail(c, LSN_ERR_INVALID, "bad lsn_load_layer_nf4 arguments");
  for (int p = 0; p < NPROJ; ++p)
    if (!codes[p] || !absmax[p]) return fail(c, LSN_ERR_INVALID, "null projection %d", p);
  std::vector<uint8_t> tmp;
  uint8_t* rec;
  if (c->cfg.mode == LSN_STREAM_FILE) {
    tmp.assign(c->rec_bytes, 0);
    rec = tmp.data();
  } else {
    // a copy queued by the last pass may still be reading the old record
    HIPCHK(c, hipStreamSynchronize(c->copy));
    rec = c->store + (uint64_t)layer * c->rec_bytes;
    memset(rec, 0, c->rec_bytes);
  }
  for (int p = 0; p < NPROJ; ++p) {
    const uint64_t n = (uint64_t)c->N[p] * c->K[p];
    memcpy(rec + c->code_off[p], codes[p], n / 2);
    memcpy(rec + c->amax_off[p], absmax[p], n / 64 * 4);
  }
  const int H = c->cfg.hidden;
  memcpy(rec + c->norm_off[0], attn_norm, H * 2);
  memcpy(rec + c->norm_off[1], mlp_norm, H * 2);
  if (c->cfg.mode == LSN_STREAM_FILE) {
    uint64_t done = 0;
    const uint64_t off = (uint64_t)layer * c->rec_bytes;
    while (done < c->rec_bytes) {
      const ssize_t w = pwrite(c->fd, rec + done, c->rec_bytes - done, off + done);
      if (w <= 0) return fail(c, LSN_ERR_IO, "write of layer %d record failed", layer);
      done += (uint64_t)w;
    }
  } else if (c->cfg.mode == LSN_RESIDENT) {
    HIPCHK(c, hipMemcpyAsync(c->records + (uint64_t)layer * c->rec_bytes, rec, c->rec_bytes,
                             hipMemcpyHostToDevice, c->cs));
    HIPCHK(c, hipStreamSynchronize(c->cs));
  }
  // a slot or staging buffer holding an older copy of this layer is stale now
  c->sched.forget(layer);
  reader_forget(c, layer);
  c->loaded[layer] = 1;
  return LSN_OK;
}

lsn_status lsn_load_head(lsn_ctx* c, const uint16_t* embed, const uint16_t* lm_head,
                         const uint16_t* final_norm) {
  CHECK_CTX(c);
  if (!embed || !final_norm || (!c->cfg.tied_embeddings && !lm_head))
    return fail(c, LSN_ERR_INVALID, "bad lsn_load_head arguments");
  const uint64_t vb = (uint64_t)c->cfg.vocab * c->cfg.hidden * 2;
  if (c->cfg.head_on_host) {
    // pinned host copies, read by the kernels through device-visible pointers
    if (!c->embed_h) {
      if (hipHostMalloc((void**)&c->embed_h, vb, hipHostMallocDefault) != hipSuccess)
        return fail(c, LSN_ERR_HIP, "pinned host embedding table");
      if (!c->cfg.tied_embeddings &&
          hipHostMalloc((void**)&c->lm_head_h, vb, hipHostMallocDefault) != hipSuccess)
        return fail(c, LSN_ERR_HIP, "pinned host LM-head table");
      if (c->cfg.tied_embeddings) c->lm_head_h = c->embed_h;
      HIPCHK(c, hipHostGetDevicePointer((void**)&c->embed, c->embed_h, 0));
      HIPCHK(c, hipHostGetDevicePointer((void**)&c->lm_head, c->lm_head_h, 0));
    }
    HIPCHK(c, hipStreamSynchronize(c->cs));  // no kernel or copy still reads the old tables
    HIPCHK(c, hipStreamSynchronize(c->copy));
    memcpy(c->embed_h, embed, vb);
    if (!c->cfg.tied_embeddings) memcpy(c->lm_head_h, lm_head, vb);
  } else {
    HIPCHK(c, hipStreamSynchronize(c->cs));  // no queued kernel still reads the old tables
    HIPCHK(c, hipMemcpy(c->embed, embed, vb, hipMemcpyHostToDevice));
    if (!c->cfg.tied_embeddings)
      HIPCHK(c, hipMemcpy(c->lm_head, lm_head, vb, hipMemcpyHostToDevice));
  }
  HIPCHK(c, hipMemcpy(c->final_norm, final_norm, (uint64_t)c->cfg.hidden * 2,
                      hipMemcpyHostToDevice));
  c->head_loaded = true;
  return LSN_OK;
}

lsn_status lsn_set_lora(lsn_ctx* c, int32_t layer, int32_t proj, const float* A, const float* B) {
  CHECK_CTX(c);
  if (layer < 0 || layer >= c->cfg.n_layers || proj < 0 || proj >= NPROJ || !c->targeted(proj))
    return fail(c, LSN_ERR_INVALID, "no adapter at layer %d projection %d", layer, proj);
  const int r = c->cfg.lora_rank;
  HIPCHK(c, hipStreamSynchronize(c->cs));
  ++c->lora_version;
  if (A) HIPCHK(c, hipMemcpy(c->A_of(layer, proj), A, (uint64_t)c->K[proj] * r * 4, hipMemcpyHostToDevice));
  if (B) HIPCHK(c, hipMemcpy(c->B_of(layer, proj), B, (uint64_t)r * c->N[proj] * 4, hipMemcpyHostToDevice));
  return LSN_OK;
}

lsn_status lsn_get_lora(lsn_ctx* c, int32_t layer, int32_t proj, float* A, float* B, float* dA,
                        float* dB) {
  CHECK_CTX(c);
  if (layer < 0 || layer >= c->cfg.n_layers || proj < 0 || proj >= NPROJ || !c->targeted(proj))
    return fail(c, LSN_ERR_INVALID, "no adapter at layer %d projection %d", layer, proj);
  const int r = c->cfg.lora_rank;
  const uint64_t na = (uint64_t)c->K[proj] * r * 4, nbb = (uint64_t)r * c->N[proj] * 4;
  HIPCHK(c, hipStreamSynchronize(c->cs));
  if (A) HIPCHK(c, hipMemcpy(A, c->A_of(layer, proj), na, hipMemcpyDeviceToHost));
  if (B) HIPCHK(c, hipMemcpy(B, c->B_of(layer, proj), nbb, hipMemcpyDeviceToHost));
  if (dA) HIPCHK(c, hipMemcpy(dA, c->dA_of(layer, proj), na, hipMemcpyDeviceToHost));
  if (dB) HIPCHK(c, hipMemcpy(dB, c->dB_of(layer, proj), nbb, hipMemcpyDeviceToHost));
  return LSN_OK;
}

lsn_status lsn_set_adapter_enabled(lsn_ctx* c, int32_t enabled) {
  CHECK_CTX(c);
  c->adapters_on = enabled != 0;
  return LSN_OK;
}

lsn_status lsn_zero_grads(lsn_ctx* c) {
  CHECK_CTX(c);
  fill_u32(c->lora_g, 0, (int64_t)c->lora_n, c->cs);
  return launch_check(c);
}

lsn_status lsn_sgd_step(lsn_ctx* c, float lr) {
  CHECK_CTX(c);
  if (!std::isfinite(lr)) return fail(c, LSN_ERR_INVALID, "non-finite learning rate");
  if (c->lora_n) sgd(c->lora_p, c->lora_g, lr, (int64_t)c->lora_n, c->cs);
  ++c->lora_version;
  return launch_check(c);
}

lsn_status lsn_begin_pass(lsn_ctx* c, int32_t kind, int32_t n_seq, int32_t seq_len) {
  CHECK_CTX(c);
  if ((kind != LSN_PASS_FWD && kind != LSN_PASS_BWD) || n_seq <= 0 || seq_len <= 0 ||
      seq_len % 8 || seq_len > c->cfg.max_seq_len ||
      (int64_t)n_seq * seq_len > c->cfg.max_tokens)
    return fail(c, LSN_ERR_INVALID, "bad pass (kind %d, %d x %d)", kind, n_seq, seq_len);
  if (kind == LSN_PASS_BWD && !c->adapters_on)
    return fail(c, LSN_ERR_STATE, "backward needs the adapters enabled");
  const int L = c->cfg.n_layers;
  c->pass_kind = kind;
  c->n_seq = n_seq;
  c->seq_len = seq_len;
  c->T = n_seq * seq_len;
  std::vector<int> order(L);
  for (int i = 0; i < L; ++i) order[i] = (kind == LSN_PASS_FWD) ? i : L - 1 - i;
  if (c->cfg.mode == LSN_RESIDENT) {  // no copies: the order only
    c->sched.order = order;
    c->sched.slot_of.assign(L, -1);
    c->sched.pos = 0;
    return LSN_OK;
  }
  HipExec x{c};
  return sched_status(c, c->sched.begin(x, order));
}

lsn_status lsn_embed(lsn_ctx* c, const int32_t* tokens, float* h0) {
  CHECK_CTX(c);
  if (!tokens || !h0 || c->T <= 0) return fail(c, LSN_ERR_INVALID, "bad lsn_embed arguments");
  if (!c->head_loaded) return fail(c, LSN_ERR_STATE, "head tables not loaded");
  embed(tokens, c->embed, c->T, c->cfg.hidden, c->cfg.vocab, h0, c->cs);
  return launch_check(c);
}

}  // extern "C"

// Runs f(token offset) once per group of whole sequences of the pass that
// the layer workspace holds (one group when it holds them all), with the
// context's token and sequence counts set to the group's; groups in order.
template <class Fn>
static lsn_status for_groups(lsn_ctx* c, Fn f) {
  const int n = c->n_seq, T = c->T;
  const int per = (int)std::max<int64_t>(1, std::min<int64_t>(n, c->TL / c->seq_len));
  lsn_status st = LSN_OK;
  for (int s0 = 0; s0 < n && st == LSN_OK; s0 += per) {
    c->n_seq = std::min(per, n - s0);
    c->T = c->n_seq * c->seq_len;
    st = f((int64_t)s0 * c->seq_len * c->cfg.hidden);
  }
  c->n_seq = n;
  c->T = T;
  return st;
}

extern "C" {

lsn_status lsn_forward_layer(lsn_ctx* c, int32_t layer, const float* h_in, float* h_out) {
  CHECK_CTX(c);
  if (!h_in || !h_out) return fail(c, LSN_ERR_INVALID, "null activation");
  const uint8_t* rec;
  lsn_status st = layer_begin(c, LSN_PASS_FWD, layer, &rec);
  if (st != LSN_OK) return st;
  st = for_groups(c, [&](int64_t o) { return layer_forward(c, layer, rec, h_in + o, h_out + o, true); });
  if (st != LSN_OK) return st;
  return layer_end(c);
}

lsn_status lsn_forward_layer_pair(lsn_ctx* c, int32_t layer, const float* h_ref_in,
                                  float* h_ref_out, const float* h_in, float* h_out) {
  CHECK_CTX(c);
  if (!h_ref_in || !h_ref_out || !h_in || !h_out)
    return fail(c, LSN_ERR_INVALID, "null activation");
  if (h_ref_out == h_in || h_ref_out == h_out || h_out == h_ref_in)
    return fail(c, LSN_ERR_INVALID, "reference and policy activations must not overlap");
  const uint8_t* rec;
  lsn_status st = layer_begin(c, LSN_PASS_FWD, layer, &rec);
  if (st != LSN_OK) return st;
  // the same record, first without the low-rank branches (reference model),
  // then with them (policy); the kernels are the ones of lsn_forward_layer
  const bool on = c->adapters_on;
  c->adapters_on = false;
  st = for_groups(c, [&](int64_t o) {
    return layer_forward(c, layer, rec, h_ref_in + o, h_ref_out + o, true);
  });
  c->adapters_on = on;
  if (st != LSN_OK) return st;
  st = for_groups(c, [&](int64_t o) { return layer_forward(c, layer, rec, h_in + o, h_out + o, true); });
  if (st != LSN_OK) return st;
  return layer_end(c);
}

lsn_status lsn_backward_layer(lsn_ctx* c, int32_t layer, const float* h_in, const float* dh_out,
                              float* dh_in) {
  CHECK_CTX(c);
  if (!h_in || !dh_out || !dh_in) return fail(c, LSN_ERR_INVALID, "null activation");
  // the recompute and the adapter gradients both need the adapters on (they
  // may have been switched off after lsn_begin_pass)
  if (!c->adapters_on) return fail(c, LSN_ERR_STATE, "backward needs the adapters enabled");
  const uint8_t* rec;
  lsn_status st = layer_begin(c, LSN_PASS_BWD, layer, &rec);
  if (st != LSN_OK) return st;
  st = for_groups(c, [&](int64_t o) {
    return layer_backward(c, layer, rec, h_in + o, dh_out + o, dh_in + o);
  });
  if (st != LSN_OK) return st;
  return layer_end(c);
}

static lsn_status lm_logits_chunk(lsn_ctx* c, const uint16_t* W, int Vc) {
  GemmParams p = base_params(c);
  p.M = c->T; p.N = Vc; p.K = c->cfg.hidden;
  p.A = c->nf; p.lda = c->cfg.hidden;
  p.B = W; p.ldb = c->cfg.hidden;
  p.C = c->logits; p.ldc = Vc;
  HIPCHK(c, cgemm(c, p, A_BF16_K, B_BF16_K, 1));
  return LSN_OK;
}

// head_on_host: W_lm rows [v0, v0 + Vc) into slot s on the copy stream, after
// the slot's previous reader is done (the scheduler's foreign-data protocol).
static lsn_status copy_head_chunk(lsn_ctx* c, int v0, int Vc, int s) {
  uint8_t* dst = c->records + (uint64_t)s * c->rec_bytes;
  HipExec x{c};
  lsn_status st = sched_status(c, c->sched.foreign_prepare(x, s));
  if (st != LSN_OK) return st;
  const uint64_t bytes = (uint64_t)Vc * c->cfg.hidden * 2;
  inject_copy_faults(c, dst, bytes);
  HIPCHK(c, hipMemcpyAsync(dst, c->lm_head_h + (int64_t)v0 * c->cfg.hidden, bytes,
                           hipMemcpyHostToDevice, c->copy));
  HIPCHK(c, hipEventRecord(c->copy_done[s], c->copy));
  c->sched.foreign_copied(s);
  c->bytes_h2d += bytes;
  return LSN_OK;
}

// Per vocabulary chunk: logits = n W_chunk^T, then the running max and sum
// of exp over the vocabulary.  With want_grad_state the pass also keeps, in
// dnf, the expected embedding row E[t] = sum_v softmax(l_t)_v W_v: each chunk
// rescales the accumulator to the new running max (alpha) and adds
// p~ W_chunk, and the end divides by the sum.  The backward then needs no
// second pass over W_lm.
lsn_status lsn_lm_head_logprobs(lsn_ctx* c, const float* h, const int32_t* targets, float* logp,
                                int32_t want_grad_state) {
  CHECK_CTX(c);
  if (!h || !targets || !logp || c->T <= 0) return fail(c, LSN_ERR_INVALID, "bad lm_head arguments");
  if (!c->head_loaded) return fail(c, LSN_ERR_STATE, "head tables not loaded");
  const int T = c->T, V = c->cfg.vocab, H = c->cfg.hidden;
  const bool acc = want_grad_state != 0;
  // head_on_host: W_lm streams through two slots chunk by chunk, the next
  // chunk copying while this one computes; those slots' layer records are
  // overwritten (the two released earliest, whose records the next pass
  // needs last), so no layer pass may be under way
  const bool host = c->cfg.head_on_host != 0;
  if (host && c->sched.in_pass())
    return fail(c, LSN_ERR_STATE, "lm_head with head_on_host inside a layer pass");
  const int nch = (V + c->vchunk - 1) / c->vchunk;
  int hs[2] = {0, 1};
  if (host) {
    lsn_status st = sched_status(c, c->sched.foreign_slots(2, hs));
    if (st != LSN_OK) return st;
    for (int i = 0; i < std::min(nch, 2); ++i) {
      st = copy_head_chunk(c, i * c->vchunk, std::min(c->vchunk, V - i * c->vchunk), hs[i]);
      if (st != LSN_OK) return st;
    }
  }
  rmsnorm_fwd(h, c->final_norm, T, H, c->cfg.rms_eps, c->nf, c->rstdf, c->cs);
  for (int i = 0, v0 = 0; v0 < V; ++i, v0 += c->vchunk) {
    const int Vc = std::min(c->vchunk, V - v0), sl = hs[i & 1];
    const uint16_t* W = c->lm_head + (int64_t)v0 * H;
    if (host) {
      HipExec x{c};
      lsn_status st = sched_status(c, c->sched.foreign_acquire(x, sl));
      if (st != LSN_OK) return st;
      W = reinterpret_cast<const uint16_t*>(c->records + (uint64_t)sl * c->rec_bytes);
    }
    lsn_status st = lm_logits_chunk(c, W, Vc);
    if (st != LSN_OK) return st;
    if (!acc) {
      lse_chunk(c->logits, T, Vc, v0, targets, c->run_m, c->run_s, c->tlogit, v0 == 0, c->cs);
    } else {
      lse_chunk_acc(c->logits, T, Vc, v0, targets, c->run_m, c->run_s, c->tlogit, c->head_f,
                    c->dlog, v0 == 0, c->cs);
      if (v0 > 0) scale_rows(c->dnf, c->head_f, T, H, c->cs);
      GemmParams p = base_params(c);  // E~ (+)= p~ W_chunk
      p.M = T; p.N = H; p.K = Vc;
      p.A = c->dlog; p.lda = Vc;
      p.B = W; p.ldb = H;
      p.C = c->dnf; p.ldc = H;
      p.cmode = (v0 == 0) ? C_F32 : C_F32_ACC;
      HIPCHK(c, cgemm(c, p, A_BF16_K, B_BF16_R, 1));
    }
    if (host) {
      HipExec x{c};
      st = sched_status(c, c->sched.foreign_release(x, sl));
      if (st != LSN_OK) return st;
      if (i + 2 < nch) {
        const int v2 = (i + 2) * c->vchunk;
        st = copy_head_chunk(c, v2, std::min(c->vchunk, V - v2), sl);
        if (st != LSN_OK) return st;
      }
    }
  }
  lse_final(c->run_m, c->run_s, c->tlogit, targets, T, V, logp, c->lse, acc ? c->head_f : nullptr,
            c->cs);
  if (acc) scale_rows(c->dnf, c->head_f, T, H, c->cs);
  c->lm_h = h;
  c->lm_T = T;
  c->lm_grad = acc;
  return launch_check(c);
}

// dn[t] = d loss / d n[t] = sum_v dlogits_v W_v with dlogits = dlogp_t
// (onehot(y_t) - softmax) = dlogp_t (W[y_t] - E[t]); then the final RMSNorm
// backward.
lsn_status lsn_lm_head_backward(lsn_ctx* c, const float* h, const int32_t* targets,
                                const float* dlogp, float* dh) {
  CHECK_CTX(c);
  if (!h || !targets || !dlogp || !dh) return fail(c, LSN_ERR_INVALID, "bad lm_head arguments");
  if (h != c->lm_h || c->lm_T != c->T || !c->lm_grad)
    return fail(c, LSN_ERR_STATE,
                "lm_head_backward must follow lm_head_logprobs with want_grad_state on the same h");
  const int T = c->T, H = c->cfg.hidden;
  head_grad(dlogp, targets, c->lm_head, T, H, c->cfg.vocab, c->dnf, c->cs);
  rmsnorm_bwd(h, c->final_norm, c->rstdf, c->dnf, nullptr, T, H, dh, c->cs);
  c->lm_grad = false;  // the accumulator is consumed
  return launch_check(c);
}

lsn_status lsn_sft_loss(lsn_ctx* c, const float* logp, const int32_t* targets, int32_t n,
                        float* loss, float* dlogp) {
  CHECK_CTX(c);
  if (!logp || !targets || !loss || !dlogp || n <= 0)
    return fail(c, LSN_ERR_INVALID, "bad sft_loss arguments");
  sft_loss(logp, targets, n, loss, dlogp, c->cs);
  return launch_check(c);
}

lsn_status lsn_dpo_loss(lsn_ctx* c, const float* lp, const float* lr, int32_t seq_len,
                        int32_t prompt_len, float beta, float* out6, float* dlogp) {
  CHECK_CTX(c);
  if (!lp || !lr || !out6 || !dlogp || seq_len < 2 || prompt_len < 1 || prompt_len >= seq_len)
    return fail(c, LSN_ERR_INVALID, "bad dpo_loss arguments");
  pref_loss(0, lp, lr, seq_len, prompt_len, beta, 0.f, out6, dlogp, c->cs);
  return launch_check(c);
}

lsn_status lsn_pref_loss(lsn_ctx* c, int32_t kind, const float* lp, const float* lr,
                         int32_t seq_len, int32_t prompt_len, float beta, float param,
                         float* out6, float* dlogp) {
  CHECK_CTX(c);
  if (kind < LSN_LOSS_DPO || kind > LSN_LOSS_KTO || !lp || !out6 || !dlogp || seq_len < 2 ||
      prompt_len < 1 || prompt_len >= seq_len)
    return fail(c, LSN_ERR_INVALID, "bad pref_loss arguments");
  if ((kind == LSN_LOSS_DPO || kind == LSN_LOSS_KTO) && !lr)
    return fail(c, LSN_ERR_INVALID, "this loss needs reference log-probs");
  pref_loss(kind, lp, lr, seq_len, prompt_len, beta, param, out6, dlogp, c->cs);
  return launch_check(c);
}

lsn_status lsn_stats(const lsn_ctx* c, uint64_t* layer_loads, uint64_t* bytes_h2d,
                     uint64_t* ws_bytes) {
  if (!c) return LSN_ERR_INVALID;
  if (layer_loads) *layer_loads = c->sched.loads;
  if (bytes_h2d) *bytes_h2d = c->bytes_h2d;
  if (ws_bytes) *ws_bytes = c->ws_needed;
  return LSN_OK;
}

lsn_status lsn_set_profiling(lsn_ctx* c, int32_t on) {
  CHECK_CTX(c);
  if (on < 0 || on > 3) return fail(c, LSN_ERR_INVALID, "profiling mask %d", on);
  HIPCHK(c, hipStreamSynchronize(c->copy));
  HIPCHK(c, hipStreamSynchronize(c->cs));
  c->prof.clear();
  c->evnext = 0;
  c->profiling = on;
  while (c->profiling && c->evpool.size() < 16384) {
    hipEvent_t e;
    HIPCHK(c, hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
    c->evpool.push_back(e);
  }
  return LSN_OK;
}

lsn_status lsn_profile_query(lsn_ctx* c, int32_t what, int32_t a, int32_t b, int32_t tile,
                             uint64_t* count, double* work, double* ms) {
  CHECK_CTX(c);
  if (what != 0 && what != 1) return fail(c, LSN_ERR_INVALID, "bad profile kind");
  HIPCHK(c, hipStreamSynchronize(c->copy));
  HIPCHK(c, hipStreamSynchronize(c->cs));
  uint64_t n = 0;
  double w = 0, t = 0;
  for (const auto& r : c->prof) {
    if (r.what != what) continue;
    if (what == 0 && (r.a != a || r.b != b || (tile >= 0 && r.tile != tile))) continue;
    float e = 0.f;
    HIPCHK(c, hipEventElapsedTime(&e, r.e0, r.e1));
    n += 1;
    w += r.work;
    t += e;
  }
  if (count) *count = n;
  if (work) *work = w;
  if (ms) *ms = t;
  return LSN_OK;
}

lsn_status lsn_set_fault_injection(lsn_ctx* c, int32_t copy_delay_us, int32_t compute_delay_us,
                                   int32_t poison_slots) {
  CHECK_CTX(c);
  if (copy_delay_us < 0 || copy_delay_us > 100000 || compute_delay_us < 0 ||
      compute_delay_us > 100000)
    return fail(c, LSN_ERR_INVALID, "fault-injection delays must be 0..100000 us");
  c->copy_delay_us = (uint32_t)copy_delay_us;
  c->compute_delay_us = (uint32_t)compute_delay_us;
  c->poison_slots = poison_slots != 0;
  return LSN_OK;
}

lsn_status lsn_copy_stream(const lsn_ctx* c, void** s) {
  if (!c || !s) return LSN_ERR_INVALID;
  *s = (void*)c->copy;
  return LSN_OK;
}

}  // extern "C"
