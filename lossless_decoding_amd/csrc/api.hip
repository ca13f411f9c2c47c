// liborthrus C ABI: argument checks, buffer carving, weight packing, and the
// orchestration of the two passes of a draft/verify step (see orthrus.h for
// the contract of every entry point).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "internal.h"

namespace {

thread_local int g_last_hip = 0;

constexpr int kAlign = 256;

inline uint64_t al(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// KV slots per (sequence, KV head): max_ctx rounded up to whole 64-key tiles
inline int kv_slots(int max_ctx) { return round_up(max_ctx, 64); }

enum { ST_IDLE = 0, ST_DRAFTED = 1, ST_VERIFIED = 2 };

// canonical tensor numel (see orthrus_weight_tensor)
uint64_t canon_numel(const orthrus_config& c, int t) {
  uint64_t d = c.d_model, qd = (uint64_t)c.n_q_heads * c.head_dim,
           kd = (uint64_t)c.n_kv_heads * c.head_dim;
  if (t == 0 || t == 1) return (uint64_t)c.vocab * d;
  if (t == 2 || t == 3) return d;
  switch ((t - 4) % 17) {
    case 0: case 1: return d;
    case 2: case 8: return qd * d;
    case 3: case 4: case 9: case 10: return kd * d;
    case 5: case 11: return d * qd;
    case 6: case 7: case 12: case 13: return (uint64_t)c.head_dim;
    case 14: case 15: return (uint64_t)c.ffn_dim * d;
    case 16: return d * (uint64_t)c.ffn_dim;
  }
  return 0;
}

int n_tensors(const orthrus_config& c) { return 4 + 17 * c.n_layers; }

uint64_t canon_offset(const orthrus_config& c, int t) {
  uint64_t o = 0;
  for (int i = 0; i < t; ++i) o += (canon_numel(c, i) + 255) / 256 * 256;
  return o;
}

struct Layout {
  // element size, dims
  int esz, L, d, hq, hkv, hd, F, V, K, G, qd, kd, nqkv;
  int cap, kpad, tmax, rmax, sc, nc, qr_max, ngroups_max, pchunk;
  int draft_tpw;   // query tiles per wave of every draft-pass attention launch
  bool bf16;
  // packed offsets (bytes)
  uint64_t p_embed, p_lm, p_fnorm, p_mask;
  std::vector<uint64_t> p_anorm, p_ffnnorm, p_qn, p_kn, p_dqn, p_dkn, p_qkv, p_dqkv, p_o, p_do,
      p_gu, p_down;
  uint64_t packed_bytes;
  // workspace offsets (bytes)
  uint64_t w_dlog, w_vlog, w_dst, w_vst;   // sampling: logits and row stats of both passes
  uint64_t w_h, w_x, w_qkv, w_q, w_act, w_opart, w_ml, w_parts, w_logits, w_rope, w_i32,
      w_part, w_rpart, w_cnt, cnt_bytes, w_amax, workspace_bytes, part_bytes;
  uint64_t kv_layer_elems, kv_bytes, scr_layer_elems, scratch_bytes;
};

// Default attention key chunk for `batch` sequences of `slots` keys over
// `kv_heads` KV heads.  Each (chunk, KV head, sequence) is a workgroup that
// writes a 64 KB partial (fp32, 128 rows), which is 1/8 of the keys' bytes
// at 1024-key chunks and 1/2 at 256.  The rule (a power of two in [128,
// 4096], measured on the decode workloads): the smallest one with at most
// 64 chunks per sequence and at most 1100 workgroups, and at least 1024 keys
// whenever 1024-key chunks still give 512 workgroups (two per compute unit).
static int default_attn_chunk(int batch, int slots, int kv_heads) {
  const long pairs = (long)batch * (kv_heads > 0 ? kv_heads : 1);
  const bool long_ok = pairs * ((slots + 1023) / 1024) >= 512;
  int sc = 128;
  while (sc < 4096) {
    const long nch = (slots + sc - 1) / sc;
    if (nch <= 64 && pairs * nch <= 1100 && !(long_ok && sc < 1024)) break;
    sc *= 2;
  }
  return sc;
}

// Kernel (a) alone (one pass, every row sees every key): the smallest power
// of two in [64, 16384] with at most 64 chunks per sequence and at most 512
// (chunk, KV head, sequence) workgroups, i.e. one round of two per compute
// unit (measured: 1024 at 4 x 16384 and 16 x 4096 keys, 8192 at 16 x 32768,
// 4096 at 8 x 32768).
static int block_attn_chunk(int batch, int ctx, int kv_heads) {
  const long pairs = (long)batch * kv_heads;
  int sc = 64;
  while (sc < 16384) {
    const long nch = (ctx + sc - 1) / sc;
    if (nch <= 64 && pairs * nch <= 512) break;
    sc *= 2;
  }
  return sc;
}

int validate(const orthrus_config* c) {
  if (!c) return ORTHRUS_EINVAL;
  if (c->n_layers < 1 || c->d_model < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
      c->head_dim < 2 || c->ffn_dim < 1 || c->vocab < 2 || c->block_k < 0 || c->max_batch < 1 ||
      c->max_batch > 256 || c->max_ctx < 2)
    return ORTHRUS_EINVAL;
  if (c->n_q_heads % c->n_kv_heads) return ORTHRUS_EINVAL;
  if (c->head_dim % 2 || c->head_dim > 128) return ORTHRUS_EINVAL;
  if (!(c->rope_theta > 1.0) || !(c->rms_eps > 0.0)) return ORTHRUS_EINVAL;
  if (c->block_k > 63) return ORTHRUS_EINVAL;
  if (c->attn_chunk != 0 &&
      (c->attn_chunk < 64 || c->attn_chunk > 4096 || (c->attn_chunk & (c->attn_chunk - 1))))
    return ORTHRUS_EINVAL;
  if (c->dtype == ORTHRUS_BF16) {
    if (c->head_dim != 128) return ORTHRUS_EINVAL;
    if (c->d_model % 256 || (c->n_q_heads * c->head_dim) % 256 || c->ffn_dim % 256)
      return ORTHRUS_EINVAL;
    if (c->vocab % 128) return ORTHRUS_EINVAL;
    if (c->d_model > 8192) return ORTHRUS_EINVAL;
  } else if (c->dtype != ORTHRUS_F32) {
    return ORTHRUS_EINVAL;
  }
  return ORTHRUS_OK;
}

void make_layout(const orthrus_config& c, Layout& y) {
  y.bf16 = c.dtype == ORTHRUS_BF16;
  y.esz = y.bf16 ? 2 : 4;
  y.L = c.n_layers; y.d = c.d_model; y.hq = c.n_q_heads; y.hkv = c.n_kv_heads; y.hd = c.head_dim;
  y.F = c.ffn_dim; y.V = c.vocab; y.K = c.block_k; y.G = y.hq / y.hkv;
  y.qd = y.hq * y.hd; y.kd = y.hkv * y.hd; y.nqkv = y.qd + 2 * y.kd;
  y.cap = kv_slots(c.max_ctx);
  y.kpad = y.K > 0 ? round_up(y.K, 32) : 0;
  // prompt rows per sequence per prefill pass: about 2048 rows per pass
  // (tall GEMMs, each attention key tile shared by the pass's rows), at
  // least 32 and at most 256 per sequence
  y.pchunk = 2048 / c.max_batch;
  y.pchunk = y.pchunk < 32 ? 32 : (y.pchunk > 256 ? 256 : y.pchunk / 32 * 32);
  y.tmax = y.K + 1 > y.pchunk ? y.K + 1 : y.pchunk;
  // physical rows: draft passes pad the mask rows to a multiple of 16
  int draft_rows = round_up(c.max_batch * y.K, 16) + c.max_batch;
  int other_rows = c.max_batch * (y.K > y.pchunk ? y.K : y.pchunk);
  y.rmax = draft_rows > other_rows ? draft_rows : other_rows;
  // attention key chunk: fixed per context so that a row's result does not
  // depend on which pass computes it
  int sc = c.attn_chunk;
  if (sc == 0) sc = default_attn_chunk(c.max_batch, y.cap, c.n_kv_heads);
  y.sc = sc;
  y.nc = (y.cap + sc - 1) / sc;
  y.qr_max = y.tmax * y.G;
  // Mask rows fold the draft block into their last chunk with two query
  // tiles per wave and keep it as a separate last partial with one, which
  // changes their low bits.  The draft pass therefore takes its tile count
  // from create-time quantities only (the full cache at max_batch), so a
  // context computes every draft row the same way whatever the call's batch
  // or the host's length bound.
  y.draft_tpw = (long)c.max_batch * y.hkv * y.nc * attn_row_groups((y.K + 1) * y.G, 2) < 512 ? 1 : 2;
  {
    int ns[4] = {y.nqkv, y.d, 2 * y.F, y.V};
    y.ngroups_max = 0;
    for (int i = 0; i < 4; ++i) if (ns[i] / 128 > y.ngroups_max) y.ngroups_max = ns[i] / 128;
  }

  // ---- packed weights
  uint64_t o = 0, E = y.esz;
  auto take = [&](uint64_t bytes) { uint64_t r = o; o = al(o + bytes); return r; };
  y.p_embed = take((uint64_t)y.V * y.d * E);
  y.p_lm = take((uint64_t)y.V * y.d * E);
  y.p_fnorm = take((uint64_t)y.d * E);
  y.p_mask = take((uint64_t)y.d * E);
  for (int l = 0; l < y.L; ++l) {
    y.p_anorm.push_back(take((uint64_t)y.d * E));
    y.p_ffnnorm.push_back(take((uint64_t)y.d * E));
    y.p_qn.push_back(take((uint64_t)y.hd * E));
    y.p_kn.push_back(take((uint64_t)y.hd * E));
    y.p_dqn.push_back(take((uint64_t)y.hd * E));
    y.p_dkn.push_back(take((uint64_t)y.hd * E));
    y.p_qkv.push_back(take((uint64_t)y.nqkv * y.d * E));
    y.p_dqkv.push_back(take((uint64_t)y.nqkv * y.d * E));
    y.p_o.push_back(take((uint64_t)y.d * y.qd * E));
    y.p_do.push_back(take((uint64_t)y.d * y.qd * E));
    y.p_gu.push_back(take((uint64_t)2 * y.F * y.d * E));
    y.p_down.push_back(take((uint64_t)y.d * y.F * E));
  }
  y.packed_bytes = o;

  // ---- KV cache and block scratch
  y.kv_layer_elems = (uint64_t)c.max_batch * y.hkv * y.cap * y.hd;
  y.kv_bytes = 2 * y.L * y.kv_layer_elems * E;
  y.scr_layer_elems = (uint64_t)c.max_batch * y.hkv * y.kpad * y.hd;
  y.scratch_bytes = 2 * y.L * y.scr_layer_elems * E;

  // ---- workspace
  o = 0;
  int xw = y.d > y.qd ? y.d : y.qd;
  y.w_h = take((uint64_t)y.rmax * y.d * 4);
  // bf16 GEMM inputs are kept in fragment order: whole 16-row tiles
  const uint64_t rows16 = (uint64_t)(y.rmax + 15) / 16 * 16;
  y.w_x = take(rows16 * xw * E);
  y.w_qkv = y.bf16 ? take(0) : take((uint64_t)y.rmax * y.nqkv * 4);
  y.w_q = take((uint64_t)y.rmax * y.qd * E);
  y.w_act = take(rows16 * y.F * E);
  uint64_t part_rows = (uint64_t)c.max_batch * y.hkv * (y.nc + 1) * y.qr_max;
  y.w_opart = y.bf16 ? take(part_rows * y.hd * 4) : take(0);
  y.w_ml = y.bf16 ? take(part_rows * 2 * 4) : take(0);
  y.w_parts = y.bf16 ? take(0) : take((uint64_t)y.rmax * 8);
  y.w_logits = y.bf16 ? take(0) : take((uint64_t)y.rmax * y.V * 4);
  y.w_rope = take((uint64_t)y.cap * (y.hd / 2) * 8);
  y.w_i32 = take((uint64_t)4 * c.max_batch * 4);
  if (y.bf16) {
    // split-K partials of the narrow GEMMs (fewer than 128 column groups)
    uint64_t nmax = 0;
    int ns[4] = {y.nqkv, y.d, 2 * y.F, y.V};
    for (int i = 0; i < 4; ++i)
      if (ns[i] / 128 < 128 && (uint64_t)ns[i] > nmax) nmax = ns[i];
    // partials are kept per padded 64-row group: [8][round_up(rows, 64)][N]
    // (+1 row group: a draft launch splits its rows into two segments)
    const uint64_t rgroups = (uint64_t)(y.rmax + 63) / 64 + 1;
    y.w_part = take(8 * rgroups * 64 * nmax * 4);
    y.part_bytes = 8 * rgroups * 64 * nmax * 4;      // addressed with 32-bit offsets
    // slice partials of the residual GEMMs (O, down): [8][rows][d]
    y.w_rpart = take(8 * (uint64_t)y.rmax * (y.d > y.nqkv ? y.d : y.nqkv) * 4);
    // completion counters of the split-K GEMM column groups (+1 grid counter)
    y.cnt_bytes = (rgroups * y.ngroups_max + 1) * 4;
    y.w_cnt = take(y.cnt_bytes);
    // per-row (value, index) partials of the LM head's column groups (at
    // least 64 columns each)
    y.w_amax = take((uint64_t)y.rmax * ((y.V + 63) / 64) * 8);
  } else {
    y.w_part = y.w_rpart = y.w_cnt = y.w_amax = take(0);
    y.part_bytes = 0;
    y.cnt_bytes = 0;
  }
  // sampling at T > 0: the draft pass's logits (anchor and mask rows) must
  // outlive the verify pass, so each pass keeps its own, with (max, sum)
  const uint64_t vrows = (uint64_t)c.max_batch * y.K;
  const uint64_t drows = (uint64_t)draft_rows;
  y.w_dlog = take(drows * y.V * 4);
  y.w_vlog = take(vrows * y.V * 4);
  y.w_dst = take(drows * 8);
  y.w_vst = take(vrows * 8);
  y.workspace_bytes = o;
}

bool aligned(const void* p) { return ((uintptr_t)p % kAlign) == 0; }

}  // namespace

inline void set_rm(PassInfo& P) {
  P.RM = P.kind == PASS_DRAFT ? round_up(P.B * P.Kx, 16) : 0;
}

struct orthrus_ctx {
  orthrus_config cfg;
  Layout y;
  char* packed;
  char* kv;
  char* scr;
  char* ws;
  int state;
  int step_batch;
  int step_k;          // block size of the outstanding step (<= block_k)
  float temp;          // sampling temperature (0: greedy)
  uint64_t seed;       // Philox key of the sampling draws
  uint32_t rng_step;   // Philox counter word of the current step
  std::vector<int64_t> bound;   // host upper bound of every sequence's length
  float* dbg_logits;
  void* dbg_attn;
  int dbg_rows;
  float* dbg_resid;    // [L+1][dbg_lrows][d]: layer inputs, then the final norm's input
  float* dbg_attn32;   // [L][dbg_lrows][qd]: attention output before rounding (bf16 models)
  int dbg_lrows;
  // opt-in launch timing: event pairs around launches of the selected classes
  uint32_t tmask;
  std::vector<hipEvent_t> ev;     // 2 per pair
  std::vector<int> ev_cls;
  int ev_used;
  bool ev_dropped;           // a selected launch found the event pairs full
};

namespace {

int hip_ok(hipError_t e) {
  if (e != hipSuccess) { g_last_hip = (int)e; return ORTHRUS_EHIP; }
  return ORTHRUS_OK;
}

int check_launch() { return hip_ok(hipGetLastError()); }

// timing classes: pass * 8 + role
enum { R_QKV = 0, R_ATTN = 1, R_O = 2, R_GU = 3, R_DOWN = 4, R_LM = 5, R_SMALL = 6, R_ACC = 7 };
inline int pass_base(int kind) { return kind * 8; }

// Times the launches in its scope with a pair of events on the stream.  The
// gate/up role is one GEMM kernel: there the kernel's dispatch records the
// pair itself (no gap from event records around it), as profiler traces do.
struct Tick {
  orthrus_ctx* c; int i; hipStream_t s; bool ext;
  Tick(orthrus_ctx* c_, int cls, hipStream_t s_) : c(c_), i(-1), s(s_), ext(false) {
    if (!(c->tmask >> cls & 1u)) return;
    if (c->ev_used * 2 >= (int)c->ev.size()) { c->ev_dropped = true; return; }
    i = c->ev_used++;
    c->ev_cls[i] = cls;
    ext = cls % 8 == R_GU;
    if (ext) gemm_time_next_launch(c->ev[2 * i], c->ev[2 * i + 1]);
    else (void)hipEventRecord(c->ev[2 * i], s);
  }
  ~Tick() {
    if (i < 0) return;
    if (!ext) { (void)hipEventRecord(c->ev[2 * i + 1], s); return; }
    if (gemm_time_pending()) {        // no GEMM launched: an empty interval
      gemm_time_next_launch(nullptr, nullptr);
      (void)hipEventRecord(c->ev[2 * i], s);
      (void)hipEventRecord(c->ev[2 * i + 1], s);
    }
  }
};

// Per-layer parity tap: residual rows of the pass (the input of layer l, or
// of the final norm for l = L) copied out when the pass fits the tap.
void tap_resid(orthrus_ctx* c, int l, const float* h, int rows, hipStream_t s) {
  if (!c->dbg_resid || rows > c->dbg_lrows) return;
  const uint64_t d = c->y.d;
  (void)hipMemcpyAsync(c->dbg_resid + (uint64_t)l * c->dbg_lrows * d, h, rows * d * 4,
                       hipMemcpyDeviceToDevice, s);
}

template <typename T> T* W(orthrus_ctx* c, uint64_t off) { return (T*)(c->packed + off); }
template <typename T> T* S(orthrus_ctx* c, uint64_t off);

SampleArgs sample_args(orthrus_ctx* c, int B, int k) {
  SampleArgs a{};
  a.T = c->temp; a.seed = c->seed; a.step = c->rng_step; a.V = c->y.V;
  a.RM = round_up(B * k, 16);
  a.dlogits = S<float>(c, c->y.w_dlog); a.vlogits = S<float>(c, c->y.w_vlog);
  a.dstats = S<float2>(c, c->y.w_dst); a.vstats = S<float2>(c, c->y.w_vst);
  return a;
}

// The logits buffer of a pass's LM head when sampling (nullptr: greedy).
float* sampling_logits(orthrus_ctx* c, const PassInfo& P) {
  if (!(c->temp > 0.f)) return nullptr;
  if (P.kind == PASS_DRAFT) return S<float>(c, c->y.w_dlog);
  if (P.kind == PASS_VERIFY) return S<float>(c, c->y.w_vlog);
  return nullptr;
}

// After a sampling pass's LM head: the debug copy of its logits, each row's
// (max, sum), the draws of a draft pass's mask rows, and for the prefill's
// last rows the first generated token.
void sample_after_lm_head(orthrus_ctx* c, const PassInfo& P, const float* slog, int32_t* drafts,
                          int32_t* pending, hipStream_t s) {
  const Layout& y = c->y;
  const int rows = P.rows();
  if (c->dbg_logits && rows <= c->dbg_rows)
    (void)hipMemcpyAsync(c->dbg_logits, slog, (uint64_t)rows * y.V * 4, hipMemcpyDeviceToDevice, s);
  SampleArgs a = sample_args(c, P.B, P.Kx);
  float2* st = S<float2>(c, P.kind == PASS_DRAFT ? y.w_dst : y.w_vst);
  launch_sample_rows(a, P, slog, y.V, st, P.kind == PASS_DRAFT ? drafts : nullptr, y.K, s);
  if (pending) launch_sample_first(a, P.B, P.RM, slog, st, pending, s);
}
template <typename T> T* S(orthrus_ctx* c, uint64_t off) { return (T*)(c->ws + off); }

// fp32 GEMM on canonical row-major weights (check models)
void gemm(orthrus_ctx* c, uint64_t woff, uint64_t woff2, const void* X, int ldx, int M, int K,
          int N, const GemmOut& o, hipStream_t s) {
  launch_gemm_f32((const float*)(c->packed + woff), (const float*)(c->packed + woff2),
                  (const float*)X, ldx, M, K, N, o, s);
}

GemmOut out_store(float* y, int ldy, int ep) {
  GemmOut o{};
  o.ep = ep; o.y = y; o.ldy = ldy;
  return o;
}

// One forward pass of the rows described by P through every layer, ending
// with the LM-head argmax when want_tokens.
void run_pass_f32(orthrus_ctx* c, const PassInfo& P, const int32_t* anchor_tok,
                  const int32_t* block_tok, int block_ld, bool want_tokens, int32_t* drafts,
                  int32_t* ar, int32_t* pending, hipStream_t s) {
  const Layout& y = c->y;
  const int rows = P.rows();
  const int BK = P.kind == PASS_DRAFT ? P.B * P.Kx : 0;   // mask rows (draft)
  const int RM = P.kind == PASS_DRAFT ? P.RM : 0;
  const int NA = P.kind == PASS_DRAFT ? P.A * P.B : 0;    // anchor rows
  const float eps = (float)c->cfg.rms_eps;
  float* h = S<float>(c, y.w_h);
  char* x = S<char>(c, y.w_x);
  float* qkv = S<float>(c, y.w_qkv);
  char* q = S<char>(c, y.w_q);
  char* act = S<char>(c, y.w_act);
  const uint64_t E = y.esz;
  const int pb = pass_base(P.kind);
  {
    Tick t(c, pb + R_SMALL, s);
    launch_embed(P, anchor_tok, block_tok, block_ld, c->packed + y.p_embed,
                 c->packed + y.p_mask, y.V, y.d, false, h, s);
  }
  for (int l = 0; l < y.L; ++l) {
    tap_resid(c, l, h, rows, s);
    launch_rmsnorm(h, rows, y.d, c->packed + y.p_anorm[l], false, eps, x, s);
    if (P.kind == PASS_DRAFT) {
      if (BK > 0)
        gemm(c, y.p_dqkv[l], 0, x, y.d, BK, y.d, y.nqkv, out_store(qkv, y.nqkv, EP_STORE), s);
      if (NA > 0)
        gemm(c, y.p_qkv[l], 0, x + (uint64_t)RM * y.d * E, y.d, NA, y.d, y.nqkv,
             out_store(qkv + (uint64_t)RM * y.nqkv, y.nqkv, EP_STORE), s);
    } else {
      gemm(c, y.p_qkv[l], 0, x, y.d, rows, y.d, y.nqkv, out_store(qkv, y.nqkv, EP_STORE), s);
    }
    char* kc = c->kv + (uint64_t)l * y.kv_layer_elems * E;
    char* vc = c->kv + ((uint64_t)y.L + l) * y.kv_layer_elems * E;
    char* ks = c->scr + (uint64_t)l * y.scr_layer_elems * E;
    char* vs = c->scr + ((uint64_t)y.L + l) * y.scr_layer_elems * E;
    launch_qkv_post(P, qkv, y.hq, y.hkv, y.hd, c->packed + y.p_qn[l], c->packed + y.p_kn[l],
                    c->packed + y.p_dqn[l], c->packed + y.p_dkn[l], false, eps,
                    S<float>(c, y.w_rope), q, kc, vc, y.cap, ks, vs, y.kpad, s);
    AttnArgs a{};
    a.P = P; a.q = q; a.kc = kc; a.vc = vc; a.cap = y.cap; a.ks = ks; a.vs = vs;
    a.kpad = y.kpad; a.hq = y.hq; a.hkv = y.hkv; a.hd = y.hd; a.sc = y.sc; a.nc = y.nc;
    a.qr_max = y.qr_max; a.out = x; a.fixed_ctx = -1;
    a.block_len = (P.kind == PASS_DRAFT) ? P.Kx : 0;
    if (c->dbg_attn && rows <= c->dbg_rows) {
      a.tap = (char*)c->dbg_attn + (uint64_t)l * c->dbg_rows * y.qd * E;
      a.tap_rows = rows;
    }
    launch_attention_f32(a, s);
    if (P.kind == PASS_DRAFT) {
      if (BK > 0) gemm(c, y.p_do[l], 0, x, y.qd, BK, y.qd, y.d, out_store(h, y.d, EP_RESID), s);
      if (NA > 0)
        gemm(c, y.p_o[l], 0, x + (uint64_t)RM * y.qd * E, y.qd, NA, y.qd, y.d,
             out_store(h + (uint64_t)RM * y.d, y.d, EP_RESID), s);
    } else {
      gemm(c, y.p_o[l], 0, x, y.qd, rows, y.qd, y.d, out_store(h, y.d, EP_RESID), s);
    }
    launch_rmsnorm(h, rows, y.d, c->packed + y.p_ffnnorm[l], false, eps, x, s);
    GemmOut og{};
    og.ep = EP_SWIGLU; og.act = act; og.ldact = y.F;
    gemm(c, y.p_gu[l], y.p_gu[l] + (uint64_t)y.F * y.d * E, x, y.d, rows, y.d, y.F, og, s);
    gemm(c, y.p_down[l], 0, act, y.F, rows, y.F, y.d, out_store(h, y.d, EP_RESID), s);
  }
  tap_resid(c, y.L, h, rows, s);
  if (!want_tokens) return;
  launch_rmsnorm(h, rows, y.d, c->packed + y.p_fnorm, false, eps, x, s);
  GemmOut ol{};
  ol.ep = EP_ARGMAX;
  ol.part = S<float2>(c, y.w_parts);
  float* slog = sampling_logits(c, P);
  ol.y = slog ? slog : S<float>(c, y.w_logits);
  ol.ldy = y.V;
  if (!slog && c->dbg_logits && rows <= c->dbg_rows) { ol.logits = c->dbg_logits; ol.ldl = y.V; }
  gemm(c, y.p_lm, 0, x, y.d, rows, y.d, y.V, ol, s);
  launch_lm_reduce(ol.part, rows, 1, P, y.K, drafts, ar, pending, s);
  if (slog) sample_after_lm_head(c, P, slog, drafts, pending, s);
}

void run_pass_bf16(orthrus_ctx* c, const PassInfo& P, const int32_t* anchor_tok,
                   const int32_t* block_tok, int block_ld, bool want_tokens, int32_t* drafts,
                   int32_t* ar, int32_t* pending, hipStream_t s) {
  const Layout& y = c->y;
  const int rows = P.rows();
  const int BK = P.kind == PASS_DRAFT ? P.B * P.Kx : 0;
  const int RM = P.kind == PASS_DRAFT ? P.RM : 0;
  const int NA = P.kind == PASS_DRAFT ? P.A * P.B : 0;
  const float eps = (float)c->cfg.rms_eps;
  float* h = S<float>(c, y.w_h);
  uint16_t* x = S<uint16_t>(c, y.w_x);   // RMSNorm output (ld d) / attention output (ld qd)
  uint16_t* q = S<uint16_t>(c, y.w_q);
  uint16_t* act = S<uint16_t>(c, y.w_act);
  const int pb = pass_base(P.kind);
  // host-side upper bound on the cache slots a sequence of the pass reaches:
  // a launch-shape hint for the attention of AR rows (prefill, anchor,
  // verify), whose results do not depend on it; draft passes take their
  // launch shape from the context instead (see draft_tpw)
  int reach = 0;
  if (P.kind == PASS_PREFILL) {
    reach = P.p0 + P.Kx;
  } else {
    for (int b = 0; b < P.B; ++b) reach = c->bound[b] + P.Kx + 1 > reach ? c->bound[b] + P.Kx + 1 : reach;
  }
  const int active_chunks = (reach + y.sc - 1) / y.sc;
  {
    Tick t(c, pb + R_SMALL, s);
    launch_embed(P, anchor_tok, block_tok, block_ld, c->packed + y.p_embed,
                 c->packed + y.p_mask, y.V, y.d, true, h, s);
  }
  GemmArgs g0{};
  g0.part = S<float>(c, y.w_part);
  g0.cnt = S<unsigned>(c, y.w_cnt);
  g0.eps = eps;
  g0.P = P; g0.hq = y.hq; g0.hkv = y.hkv;
  g0.rope = S<float2>(c, y.w_rope); g0.q_out = q; g0.cap = y.cap; g0.kpad = y.kpad;
  // residual add of the O / down slice partials (nsl = 8 when those GEMMs
  // split K; otherwise they added into h themselves) and the RMSNorm that
  // produces the next GEMM's bf16 input
  float* rpart = S<float>(c, y.w_rpart);
  const size_t rps = (size_t)y.rmax * (y.d > y.nqkv ? y.d : y.nqkv);   // slice stride
  auto rnorm = [&](int nsl, uint64_t gain_off) {
    Tick t(c, pb + R_SMALL, s);
    launch_resid_norm_bf16(P, h, y.d, rpart, rps, nsl, (const uint16_t*)(c->packed + gain_off),
                           eps, x, s);
  };
  g0.rpart = rpart; g0.rps = rps;
  tap_resid(c, 0, h, rows, s);
  rnorm(0, y.p_anorm[0]);
  auto run = [&](GemmArgs g, uint64_t w, int row0, int M, int K, int N, int ep) {
    g.W = (const u32x4_t*)(c->packed + w);
    g.row0 = row0; g.M = M; g.K = K; g.N = N; g.ep = ep;
    launch_gemm_bf16(g, s);
  };
  // draft: mask rows [0, BK) with the diffusion weights and the anchor rows
  // [RM, RM + NA) with the frozen ones, one launch
  auto run2 = [&](GemmArgs g, uint64_t wd, uint64_t wf, int K, int N, int ep) {
    g.W = (const u32x4_t*)(c->packed + wd); g.row0 = 0; g.M = BK;
    g.W2 = (const u32x4_t*)(c->packed + wf); g.row02 = RM; g.M2 = NA;
    g.K = K; g.N = N; g.ep = ep;
    launch_gemm_bf16(g, s);
  };
  for (int l = 0; l < y.L; ++l) {
    const uint64_t E = 2;
    uint16_t* kc = (uint16_t*)(c->kv + (uint64_t)l * y.kv_layer_elems * E);
    uint16_t* vc = (uint16_t*)(c->kv + ((uint64_t)y.L + l) * y.kv_layer_elems * E);
    uint16_t* ks = (uint16_t*)(c->scr + (uint64_t)l * y.scr_layer_elems * E);
    uint16_t* vs = (uint16_t*)(c->scr + ((uint64_t)y.L + l) * y.scr_layer_elems * E);
    // RMSNorm, then Q/K/V projection + QK-norm + RoPE + K/V placement; mask
    // rows use the diffusion projections, every other row the frozen ones
    {
      Tick t(c, pb + R_QKV, s);
      GemmArgs g = g0;
      g.X = x; g.ldx = y.d;
      g.qn = (const uint16_t*)(c->packed + y.p_qn[l]);
      g.kn = (const uint16_t*)(c->packed + y.p_kn[l]);
      g.dqn = (const uint16_t*)(c->packed + y.p_dqn[l]);
      g.dkn = (const uint16_t*)(c->packed + y.p_dkn[l]);
      g.kc = kc; g.vc = vc; g.ks = ks; g.vs = vs;
      if (P.kind == PASS_DRAFT && NA > 0 && gemm_bf16_rows_form(BK, y.nqkv, EP_QKV)) {
        // many mask rows: their own row-split launch (wider column groups than
        // a two-segment one) and a small launch for the anchor rows; every
        // row's arithmetic is the same in either form.  When both write slice
        // partials (disjoint rows of the partial buffer), one finish kernel
        // takes both row ranges.
        const bool one_finish = gemm_bf16_split_slices(BK, 0, y.nqkv, EP_QKV) > 0 &&
                                gemm_bf16_split_slices(NA, 0, y.nqkv, EP_QKV) > 0;
        g.defer_finish = one_finish;
        run(g, y.p_dqkv[l], 0, BK, y.d, y.nqkv, EP_QKV);
        run(g, y.p_qkv[l], RM, NA, y.d, y.nqkv, EP_QKV);
        if (one_finish) {
          g.row0 = 0; g.M = BK; g.row02 = RM; g.M2 = NA; g.N = y.nqkv;
          launch_qkv_finish_bf16(g, s);
        }
      } else if (P.kind == PASS_DRAFT) {
        run2(g, y.p_dqkv[l], y.p_qkv[l], y.d, y.nqkv, EP_QKV);
      } else {
        run(g, y.p_qkv[l], 0, rows, y.d, y.nqkv, EP_QKV);
      }
    }
    AttnArgs a{};
    a.P = P; a.q = q; a.kc = kc; a.vc = vc; a.cap = y.cap; a.ks = ks; a.vs = vs;
    a.kpad = y.kpad; a.hq = y.hq; a.hkv = y.hkv; a.hd = y.hd; a.sc = y.sc; a.nc = y.nc;
    a.qr_max = y.qr_max; a.opart = S<float>(c, y.w_opart); a.ml = S<float>(c, y.w_ml);
    a.out = x; a.out_kb = y.qd / 32;   // the O projection's input, fragment order
    a.fixed_ctx = -1; a.block_len = (P.kind == PASS_DRAFT) ? P.Kx : 0;
    a.active_chunks = active_chunks;
    if (P.kind == PASS_DRAFT && P.Kx > 0) a.tpw = y.draft_tpw;
    if (c->dbg_attn && rows <= c->dbg_rows) {
      a.tap = (char*)c->dbg_attn + (uint64_t)l * c->dbg_rows * y.qd * 2;
      a.tap_rows = rows;
    }
    if (c->dbg_attn32 && rows <= c->dbg_lrows) {
      a.tap32 = c->dbg_attn32 + (uint64_t)l * c->dbg_lrows * y.qd;
      a.tap32_rows = rows;
    }
    {
      Tick t(c, pb + R_ATTN, s);
      launch_attention_bf16(a, s);
    }
    // O projection (slice partials), then residual + FFN RMSNorm
    {
      Tick t(c, pb + R_O, s);
      GemmArgs g = g0;
      g.X = x; g.ldx = y.qd; g.y = h; g.ldy = y.d;
      if (P.kind == PASS_DRAFT) {
        run2(g, y.p_do[l], y.p_o[l], y.qd, y.d, EP_RESID);
      } else {
        run(g, y.p_o[l], 0, rows, y.qd, y.d, EP_RESID);
      }
    }
    rnorm(P.kind == PASS_DRAFT ? gemm_bf16_split_slices(BK, NA, y.d, EP_RESID)
                               : gemm_bf16_split_slices(rows, 0, y.d, EP_RESID), y.p_ffnnorm[l]);
    {
      Tick t(c, pb + R_GU, s);
      GemmArgs g = g0;
      g.X = x; g.ldx = y.d;
      g.act = act; g.ldact = y.F;
      run(g, y.p_gu[l], 0, rows, y.d, 2 * y.F, EP_SWIGLU);
    }
    {
      Tick t(c, pb + R_DOWN, s);
      GemmArgs g = g0;
      g.X = act; g.ldx = y.F; g.y = h; g.ldy = y.d;
      run(g, y.p_down[l], 0, rows, y.F, y.d, EP_RESID);
    }
    // residual + the next RMSNorm: the next layer's attention norm, or the
    // final norm in front of the LM head
    rnorm(gemm_bf16_split_slices(rows, 0, y.d, EP_RESID), l + 1 < y.L ? y.p_anorm[l + 1] : y.p_fnorm);
    tap_resid(c, l + 1, h, rows, s);
  }
  if (!want_tokens) return;
  Tick tl(c, pb + R_LM, s);
  GemmArgs g = g0;
  g.X = x; g.ldx = y.d;
  g.amax = S<float2>(c, y.w_amax);
  g.Kb = y.K; g.drafts = drafts; g.ar = ar; g.pending = pending;
  float* slog = sampling_logits(c, P);
  if (slog) { g.logits = slog; g.ldl = y.V; }
  else if (c->dbg_logits && rows <= c->dbg_rows) { g.logits = c->dbg_logits; g.ldl = y.V; }
  run(g, y.p_lm, 0, rows, y.d, y.V, EP_ARGMAX);
  if (slog) sample_after_lm_head(c, P, slog, drafts, pending, s);
}

void run_pass(orthrus_ctx* c, const PassInfo& P, const int32_t* anchor_tok,
              const int32_t* block_tok, int block_ld, bool want_tokens, int32_t* drafts,
              int32_t* ar, int32_t* pending, hipStream_t s) {
  if (c->y.bf16) run_pass_bf16(c, P, anchor_tok, block_tok, block_ld, want_tokens, drafts, ar,
                               pending, s);
  else run_pass_f32(c, P, anchor_tok, block_tok, block_ld, want_tokens, drafts, ar, pending, s);
}

}  // namespace

extern "C" {

int orthrus_query_sizes(const orthrus_config* cfg, orthrus_sizes* out) {
  int rc = validate(cfg);
  if (rc) return rc;
  if (!out) return ORTHRUS_EINVAL;
  Layout y;
  make_layout(*cfg, y);
  if (y.part_bytes >= (1ull << 31)) return ORTHRUS_EINVAL;   // batch too large for one context
  out->weights_bytes = canon_offset(*cfg, n_tensors(*cfg)) * y.esz;
  out->packed_bytes = y.packed_bytes;
  out->kv_bytes = y.kv_bytes;
  out->scratch_bytes = y.scratch_bytes;
  out->workspace_bytes = y.workspace_bytes;
  out->kv_slots = (uint64_t)y.cap;
  out->prefill_rows = (uint64_t)y.pchunk;
  return ORTHRUS_OK;
}

int orthrus_weight_tensor(const orthrus_config* cfg, int32_t index, uint64_t* offset_elems,
                          uint64_t* numel) {
  int rc = validate(cfg);
  if (rc) return rc;
  if (!offset_elems || !numel) return ORTHRUS_EINVAL;
  int nt = n_tensors(*cfg);
  if (index == -1) { *offset_elems = 0; *numel = canon_offset(*cfg, nt); return ORTHRUS_OK; }
  if (index < 0 || index >= nt) return ORTHRUS_EINVAL;
  *offset_elems = canon_offset(*cfg, index);
  *numel = canon_numel(*cfg, index);
  return ORTHRUS_OK;
}

int orthrus_create(const orthrus_config* cfg, const void* weights, void* packed, void* kv_cache,
                   void* block_scratch, void* workspace, void* stream, orthrus_ctx** out) {
  int rc = validate(cfg);
  if (rc) return rc;
  if (!out || !weights || !packed || !kv_cache || !workspace) return ORTHRUS_EINVAL;
  if (cfg->block_k > 0 && !block_scratch) return ORTHRUS_EINVAL;
  if (!aligned(weights) || !aligned(packed) || !aligned(kv_cache) || !aligned(workspace) ||
      (block_scratch && !aligned(block_scratch)))
    return ORTHRUS_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  orthrus_ctx* c = new orthrus_ctx();
  c->cfg = *cfg;
  make_layout(*cfg, c->y);
  if (c->y.part_bytes >= (1ull << 31)) { delete c; return ORTHRUS_EINVAL; }
  c->packed = (char*)packed; c->kv = (char*)kv_cache; c->scr = (char*)block_scratch;
  c->ws = (char*)workspace;
  c->state = ST_IDLE; c->step_batch = 0; c->step_k = 0;
  c->temp = 0.f; c->seed = 0; c->rng_step = 0;
  c->bound.assign(cfg->max_batch, 0);
  c->dbg_logits = nullptr; c->dbg_attn = nullptr; c->dbg_rows = 0;
  c->dbg_resid = nullptr; c->dbg_attn32 = nullptr; c->dbg_lrows = 0;
  c->tmask = 0; c->ev_used = 0; c->ev_dropped = false;
  const Layout& y = c->y;
  const uint64_t E = y.esz;
  const char* w = (const char*)weights;
  auto src = [&](int t) { return w + canon_offset(*cfg, t) * E; };
  auto copy = [&](uint64_t dst, int t) {
    return hipMemcpyAsync(c->packed + dst, src(t), canon_numel(*cfg, t) * E,
                          hipMemcpyDeviceToDevice, s);
  };
  hipError_t e = hipSuccess;
  auto chk = [&](hipError_t x) { if (x != hipSuccess && e == hipSuccess) e = x; };
  chk(copy(y.p_embed, 0));
  chk(copy(y.p_fnorm, 2));
  chk(copy(y.p_mask, 3));
  if (y.bf16) launch_pack_bf16((const uint16_t*)src(1), y.V, y.d, c->packed + y.p_lm, 0, 1, s);
  else chk(copy(y.p_lm, 1));
  for (int l = 0; l < y.L; ++l) {
    int b0 = 4 + 17 * l;
    chk(copy(y.p_anorm[l], b0 + 0));
    chk(copy(y.p_ffnnorm[l], b0 + 1));
    chk(copy(y.p_qn[l], b0 + 6));
    chk(copy(y.p_kn[l], b0 + 7));
    chk(copy(y.p_dqn[l], b0 + 12));
    chk(copy(y.p_dkn[l], b0 + 13));
    if (y.bf16) {
      const int KBd = y.d / 32;
      auto pack_rows = [&](uint64_t dst, int t, int N, int K, int nb_off, int nb_stride) {
        launch_pack_bf16((const uint16_t*)src(t), N, K, c->packed + dst, nb_off, nb_stride, s);
      };
      (void)KBd;
      // [Wq; Wk; Wv] -> one packed matrix of nqkv output rows
      pack_rows(y.p_qkv[l], b0 + 2, y.qd, y.d, 0, 1);
      pack_rows(y.p_qkv[l], b0 + 3, y.kd, y.d, y.qd / 16, 1);
      pack_rows(y.p_qkv[l], b0 + 4, y.kd, y.d, (y.qd + y.kd) / 16, 1);
      pack_rows(y.p_dqkv[l], b0 + 8, y.qd, y.d, 0, 1);
      pack_rows(y.p_dqkv[l], b0 + 9, y.kd, y.d, y.qd / 16, 1);
      pack_rows(y.p_dqkv[l], b0 + 10, y.kd, y.d, (y.qd + y.kd) / 16, 1);
      pack_rows(y.p_o[l], b0 + 5, y.d, y.qd, 0, 1);
      pack_rows(y.p_do[l], b0 + 11, y.d, y.qd, 0, 1);
      // gate block j -> packed block 2j, up block j -> 2j+1
      pack_rows(y.p_gu[l], b0 + 14, y.F, y.d, 0, 2);
      pack_rows(y.p_gu[l], b0 + 15, y.F, y.d, 1, 2);
      pack_rows(y.p_down[l], b0 + 16, y.d, y.F, 0, 1);
    } else {
      uint64_t qb = (uint64_t)y.qd * y.d * E, kb = (uint64_t)y.kd * y.d * E;
      chk(hipMemcpyAsync(c->packed + y.p_qkv[l], src(b0 + 2), qb, hipMemcpyDeviceToDevice, s));
      chk(hipMemcpyAsync(c->packed + y.p_qkv[l] + qb, src(b0 + 3), kb, hipMemcpyDeviceToDevice, s));
      chk(hipMemcpyAsync(c->packed + y.p_qkv[l] + qb + kb, src(b0 + 4), kb,
                         hipMemcpyDeviceToDevice, s));
      chk(hipMemcpyAsync(c->packed + y.p_dqkv[l], src(b0 + 8), qb, hipMemcpyDeviceToDevice, s));
      chk(hipMemcpyAsync(c->packed + y.p_dqkv[l] + qb, src(b0 + 9), kb, hipMemcpyDeviceToDevice, s));
      chk(hipMemcpyAsync(c->packed + y.p_dqkv[l] + qb + kb, src(b0 + 10), kb,
                         hipMemcpyDeviceToDevice, s));
      chk(copy(y.p_o[l], b0 + 5));
      chk(copy(y.p_do[l], b0 + 11));
      uint64_t fb = (uint64_t)y.F * y.d * E;
      chk(hipMemcpyAsync(c->packed + y.p_gu[l], src(b0 + 14), fb, hipMemcpyDeviceToDevice, s));
      chk(hipMemcpyAsync(c->packed + y.p_gu[l] + fb, src(b0 + 15), fb, hipMemcpyDeviceToDevice, s));
      chk(copy(y.p_down[l], b0 + 16));
    }
  }
  // RoPE table: angle pos * theta^(-2i/hd) in float64, stored as fp32 (cos, sin)
  std::vector<float> rope((size_t)y.cap * y.hd);
  for (int p = 0; p < y.cap; ++p)
    for (int i = 0; i < y.hd / 2; ++i) {
      double ang = (double)p * pow(cfg->rope_theta, -2.0 * i / y.hd);
      rope[((size_t)p * (y.hd / 2) + i) * 2] = (float)cos(ang);
      rope[((size_t)p * (y.hd / 2) + i) * 2 + 1] = (float)sin(ang);
    }
  chk(hipMemcpyAsync(c->ws + y.w_rope, rope.data(), rope.size() * 4, hipMemcpyHostToDevice, s));
  if (y.cnt_bytes) chk(hipMemsetAsync(c->ws + y.w_cnt, 0, y.cnt_bytes, s));
  chk(hipGetLastError());
  chk(hipStreamSynchronize(s));
  if (e != hipSuccess) {
    g_last_hip = (int)e;
    delete c;
    return ORTHRUS_EHIP;
  }
  *out = c;
  return ORTHRUS_OK;
}

int orthrus_destroy(orthrus_ctx* ctx) {
  if (!ctx) return ORTHRUS_EINVAL;
  for (hipEvent_t e : ctx->ev) (void)hipEventDestroy(e);
  delete ctx;
  return ORTHRUS_OK;
}

int orthrus_set_debug(orthrus_ctx* ctx, float* logits, void* attn, int32_t rows_cap) {
  if (!ctx || rows_cap < 0) return ORTHRUS_EINVAL;
  if ((logits || attn) && rows_cap == 0) return ORTHRUS_EINVAL;
  ctx->dbg_logits = logits;
  ctx->dbg_attn = attn;
  ctx->dbg_rows = rows_cap;
  return ORTHRUS_OK;
}

int orthrus_set_sampling(orthrus_ctx* ctx, float temperature, uint64_t seed) {
  if (!ctx || !(temperature >= 0.f) || !(temperature <= 1e4f)) return ORTHRUS_EINVAL;
  if (ctx->state != ST_IDLE) return ORTHRUS_ESTATE;
  ctx->temp = temperature;
  ctx->seed = seed;
  ctx->rng_step = 0;
  return ORTHRUS_OK;
}

int orthrus_set_debug_layers(orthrus_ctx* ctx, float* resid, float* attn32, int32_t rows_cap) {
  if (!ctx || rows_cap < 0) return ORTHRUS_EINVAL;
  if ((resid || attn32) && rows_cap == 0) return ORTHRUS_EINVAL;
  if (attn32 && !ctx->y.bf16) return ORTHRUS_EINVAL;
  ctx->dbg_resid = resid;
  ctx->dbg_attn32 = attn32;
  ctx->dbg_lrows = rows_cap;
  return ORTHRUS_OK;
}

int orthrus_prefill(orthrus_ctx* ctx, int32_t batch, const int32_t* tokens, int32_t tokens_stride,
                    const int32_t* prompt_len, int32_t max_prompt_len, int32_t* seq_len,
                    int32_t* pending, void* stream) {
  if (!ctx || !tokens || !prompt_len || !seq_len || !pending) return ORTHRUS_EINVAL;
  if (batch < 1 || batch > ctx->cfg.max_batch || tokens_stride < 1) return ORTHRUS_EINVAL;
  const int pmax = max_prompt_len;
  if (pmax < 1 || pmax > tokens_stride) return ORTHRUS_EINVAL;
  // prefill rows of every sequence run to pmax-1 (rows past a sequence's own
  // prompt compute values that land in slots no later step reads)
  if (pmax + 1 > ctx->y.cap || pmax > ctx->cfg.max_ctx) return ORTHRUS_ECAPACITY;
  hipStream_t s = (hipStream_t)stream;
  const Layout& y = ctx->y;
  int32_t* last_tok = S<int32_t>(ctx, y.w_i32) + ctx->cfg.max_batch;
  for (int p0 = 0; p0 < pmax - 1; p0 += y.pchunk) {
    PassInfo P{};
    P.kind = PASS_PREFILL; P.B = batch; P.A = 0;
    P.Kx = (pmax - 1 - p0) < y.pchunk ? (pmax - 1 - p0) : y.pchunk;
    P.p0 = p0; P.len = nullptr;
    set_rm(P);
    run_pass(ctx, P, nullptr, tokens, tokens_stride, false, nullptr, nullptr, nullptr, s);
  }
  launch_prefill_tail(batch, tokens, tokens_stride, prompt_len, pmax, seq_len, last_tok, s);
  PassInfo P{};
  P.kind = PASS_DRAFT; P.B = batch; P.A = 1; P.Kx = 0; P.p0 = 0; P.len = seq_len;
  set_rm(P);
  run_pass(ctx, P, last_tok, nullptr, 0, true, nullptr, nullptr, pending, s);
  launch_len_add(batch, seq_len, 1, s);
  int rc = check_launch();
  if (rc) return rc;
  for (int b = 0; b < ctx->cfg.max_batch; ++b) ctx->bound[b] = b < batch ? pmax : 0;
  ctx->state = ST_IDLE;
  return ORTHRUS_OK;
}

int orthrus_draft_block_k(orthrus_ctx* ctx, int32_t batch, int32_t k, const int32_t* seq_len,
                          const int32_t* pending, int32_t* drafts, int32_t* ar_tokens,
                          void* stream) {
  if (!ctx || !seq_len || !pending || !ar_tokens) return ORTHRUS_EINVAL;
  if (k < 0 || k > ctx->y.K) return ORTHRUS_EINVAL;
  if (ctx->y.K > 0 && !drafts) return ORTHRUS_EINVAL;
  if (batch < 1 || batch > ctx->cfg.max_batch) return ORTHRUS_EINVAL;
  if (ctx->state != ST_IDLE) return ORTHRUS_ESTATE;
  for (int b = 0; b < batch; ++b)
    if (ctx->bound[b] < 1) return ORTHRUS_ESTATE;          // never prefilled
  for (int b = 0; b < batch; ++b)
    if (ctx->bound[b] + k + 1 > ctx->cfg.max_ctx) return ORTHRUS_ECAPACITY;
  PassInfo P{};
  P.kind = PASS_DRAFT; P.B = batch; P.A = 1; P.Kx = k; P.p0 = 0; P.len = seq_len;
  set_rm(P);
  run_pass(ctx, P, pending, nullptr, 0, true, drafts, ar_tokens, nullptr, (hipStream_t)stream);
  int rc = check_launch();
  if (rc) return rc;
  ctx->state = ST_DRAFTED;
  ctx->step_batch = batch;
  ctx->step_k = k;
  return ORTHRUS_OK;
}

int orthrus_draft_refine(orthrus_ctx* ctx, int32_t batch, const int32_t* seq_len,
                         int32_t* drafts, void* stream) {
  if (!ctx || !seq_len || !drafts) return ORTHRUS_EINVAL;
  if (ctx->state != ST_DRAFTED) return ORTHRUS_ESTATE;
  if (batch != ctx->step_batch) return ORTHRUS_EINVAL;
  if (ctx->step_k == 0) return ORTHRUS_OK;                 // no block to refine
  PassInfo P{};
  P.kind = PASS_DRAFT; P.B = batch; P.A = 0; P.Kx = ctx->step_k; P.p0 = 0; P.len = seq_len;
  P.refine = 1;
  set_rm(P);
  run_pass(ctx, P, nullptr, drafts, ctx->y.K, true, drafts, nullptr, nullptr, (hipStream_t)stream);
  return check_launch();
}

int orthrus_draft_block(orthrus_ctx* ctx, int32_t batch, const int32_t* seq_len,
                        const int32_t* pending, int32_t* drafts, int32_t* ar_tokens,
                        void* stream) {
  if (!ctx) return ORTHRUS_EINVAL;
  return orthrus_draft_block_k(ctx, batch, ctx->y.K, seq_len, pending, drafts, ar_tokens, stream);
}

int orthrus_verify_accept(orthrus_ctx* ctx, int32_t batch, const int32_t* seq_len,
                          const int32_t* drafts, int32_t* ar_tokens, int32_t* accept_len,
                          void* stream) {
  if (!ctx || !seq_len || !ar_tokens || !accept_len) return ORTHRUS_EINVAL;
  if (ctx->y.K > 0 && !drafts) return ORTHRUS_EINVAL;
  if (ctx->state != ST_DRAFTED) return ORTHRUS_ESTATE;
  if (batch != ctx->step_batch) return ORTHRUS_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const int K = ctx->step_k;
  if (K > 0) {
    PassInfo P{};
    P.kind = PASS_VERIFY; P.B = batch; P.A = 0; P.Kx = K; P.p0 = 0; P.len = seq_len;
    set_rm(P);
    run_pass(ctx, P, nullptr, drafts, ctx->y.K, true, nullptr, ar_tokens, nullptr, s);
  }
  {
    Tick t(ctx, pass_base(PASS_VERIFY) + R_ACC, s);
    if (ctx->temp > 0.f)
      launch_spec_accept(sample_args(ctx, batch, K), batch, K, ctx->y.K, drafts, ar_tokens,
                         accept_len, s);
    else
      launch_accept(batch, K, ctx->y.K, drafts, ar_tokens, accept_len, s);
  }
  int rc = check_launch();
  if (rc) return rc;
  ctx->state = ST_VERIFIED;
  return ORTHRUS_OK;
}

int orthrus_commit_kv(orthrus_ctx* ctx, int32_t batch, const int32_t* accept_len,
                      const int32_t* ar_tokens, const int32_t* drafts, int32_t* seq_len,
                      int32_t* pending, int32_t* commit_start, int32_t* out_tokens,
                      int32_t* out_off, void* stream) {
  if (!ctx || !accept_len || !ar_tokens || !seq_len || !pending || !commit_start ||
      !out_tokens || !out_off)
    return ORTHRUS_EINVAL;
  if (ctx->y.K > 0 && !drafts) return ORTHRUS_EINVAL;
  if (ctx->state != ST_VERIFIED) return ORTHRUS_ESTATE;
  if (batch != ctx->step_batch) return ORTHRUS_EINVAL;
  {
    Tick t(ctx, pass_base(PASS_VERIFY) + R_ACC, (hipStream_t)stream);
    launch_commit(batch, ctx->y.K, accept_len, ar_tokens, drafts, seq_len, pending,
                  commit_start, out_tokens, out_off, (hipStream_t)stream);
  }
  int rc = check_launch();
  if (rc) return rc;
  for (int b = 0; b < batch; ++b) ctx->bound[b] += ctx->step_k + 1;
  ctx->rng_step += 1;
  ctx->state = ST_IDLE;
  return ORTHRUS_OK;
}

int orthrus_timing_enable(orthrus_ctx* ctx, uint32_t class_mask, int32_t capacity) {
  if (!ctx || capacity < 0) return ORTHRUS_EINVAL;
  if (class_mask && capacity == 0) return ORTHRUS_EINVAL;
  for (hipEvent_t e : ctx->ev) (void)hipEventDestroy(e);
  ctx->ev.clear(); ctx->ev_cls.clear(); ctx->ev_used = 0; ctx->ev_dropped = false; ctx->tmask = 0;
  if (!class_mask) return ORTHRUS_OK;
  ctx->ev.resize((size_t)2 * capacity);
  ctx->ev_cls.resize(capacity);
  for (auto& e : ctx->ev) {
    int rc = hip_ok(hipEventCreate(&e));
    if (rc) { e = nullptr; return rc; }
  }
  ctx->tmask = class_mask;
  return ORTHRUS_OK;
}

int orthrus_timing_read(orthrus_ctx* ctx, double* ms, int64_t* launches) {
  if (!ctx || !ms || !launches) return ORTHRUS_EINVAL;
  for (int k = 0; k < ORTHRUS_TIMING_CLASSES; ++k) { ms[k] = 0.0; launches[k] = 0; }
  for (int i = 0; i < ctx->ev_used; ++i) {
    int rc = hip_ok(hipEventSynchronize(ctx->ev[2 * i + 1]));
    if (rc) return rc;
    float t = 0.f;
    rc = hip_ok(hipEventElapsedTime(&t, ctx->ev[2 * i], ctx->ev[2 * i + 1]));
    if (rc) return rc;
    ms[ctx->ev_cls[i]] += t;
    launches[ctx->ev_cls[i]] += 1;
  }
  const bool dropped = ctx->ev_dropped;
  ctx->ev_used = 0;
  ctx->ev_dropped = false;
  return dropped ? ORTHRUS_ECAPACITY : ORTHRUS_OK;
}

int orthrus_sync_lengths(orthrus_ctx* ctx, int32_t batch, const int32_t* seq_len_host) {
  if (!ctx || !seq_len_host || batch < 1 || batch > ctx->cfg.max_batch) return ORTHRUS_EINVAL;
  if (ctx->state != ST_IDLE) return ORTHRUS_ESTATE;
  for (int b = 0; b < batch; ++b)
    if (seq_len_host[b] < 1 || seq_len_host[b] > ctx->bound[b]) return ORTHRUS_EINVAL;
  for (int b = 0; b < batch; ++b) ctx->bound[b] = seq_len_host[b];
  return ORTHRUS_OK;
}

int orthrus_reserve_steps(orthrus_ctx* ctx, int32_t batch, int32_t k, int32_t n_steps) {
  if (!ctx || batch < 1 || batch > ctx->cfg.max_batch || k < 0 || k > ctx->y.K || n_steps < 0)
    return ORTHRUS_EINVAL;
  if (ctx->state != ST_IDLE) return ORTHRUS_ESTATE;
  for (int b = 0; b < batch; ++b) {
    if (ctx->bound[b] < 1) return ORTHRUS_ESTATE;          // never prefilled
    if ((int64_t)ctx->bound[b] + (int64_t)n_steps * (k + 1) > ctx->cfg.max_ctx) return ORTHRUS_ECAPACITY;
  }
  for (int b = 0; b < batch; ++b) ctx->bound[b] += n_steps * (k + 1);
  return ORTHRUS_OK;
}

// kernel (a) alone: chunks of the cache keys, at least one (the draft block
// is streamed by the last chunk, chunk 0 when there are no cache keys)
static int block_attn_nchunks(int ctx_len, int sc) {
  const int nc = (ctx_len + sc - 1) / sc;
  return nc > 0 ? nc : 1;
}

uint64_t orthrus_attention_workspace(int32_t batch, int32_t rows, int32_t n_q_heads,
                                     int32_t n_kv_heads, int32_t ctx_len) {
  if (batch < 1 || rows < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || ctx_len < 0) return 0;
  int sc = block_attn_chunk(batch, ctx_len, n_kv_heads);
  int nc = block_attn_nchunks(ctx_len, sc);
  uint64_t qr = (uint64_t)rows * (n_q_heads / n_kv_heads);
  uint64_t pr = (uint64_t)batch * n_kv_heads * (nc + 1) * qr;
  return al(pr * 128 * 4) + al(pr * 2 * 4);
}

}  // extern "C"

namespace {

// Argument checks shared by both forms of kernel (a) alone.
int block_attention_args(int32_t batch, int32_t rows, int32_t n_q_heads, int32_t n_kv_heads,
                         const void* q, const void* k_cache, const void* v_cache, int32_t cap,
                         int32_t ctx_len, const void* k_block, const void* v_block,
                         int32_t block_len, void* out) {
  if (batch < 1 || rows < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads)
    return ORTHRUS_EINVAL;
  if (rows > 64 || cap % 64 || ctx_len < 0 || ctx_len > cap || block_len < 0 ||
      block_len > 64 || ctx_len + block_len < 1)
    return ORTHRUS_EINVAL;
  if (!q || !out || (ctx_len > 0 && (!k_cache || !v_cache)) ||
      (block_len > 0 && (!k_block || !v_block)))
    return ORTHRUS_EINVAL;
  return ORTHRUS_OK;
}

// Kernel (a) alone with its chunk partials in `workspace` (checked by the
// caller: at least orthrus_attention_workspace bytes, 256-byte aligned).
int block_attention_run(int32_t batch, int32_t rows, int32_t n_q_heads, int32_t n_kv_heads,
                        const void* q, const void* k_cache, const void* v_cache, int32_t cap,
                        int32_t ctx_len, const void* k_block, const void* v_block,
                        int32_t block_len, void* out, void* workspace, void* stream) {
  int G = n_q_heads / n_kv_heads;
  int sc = block_attn_chunk(batch, ctx_len, n_kv_heads);
  int nc = block_attn_nchunks(ctx_len, sc);
  uint64_t pr = (uint64_t)batch * n_kv_heads * (nc + 1) * rows * G;
  AttnArgs a{};
  a.P.kind = PASS_DRAFT; a.P.B = batch; a.P.A = 0; a.P.Kx = rows; a.P.p0 = 0; a.P.len = nullptr;
  a.P.RM = batch * rows;
  a.q = q; a.kc = k_cache; a.vc = v_cache; a.cap = cap; a.ks = k_block; a.vs = v_block;
  a.kpad = round_up(block_len, 32); a.hq = n_q_heads; a.hkv = n_kv_heads; a.hd = 128;
  a.sc = sc; a.nc = nc; a.qr_max = rows * G;
  a.opart = (float*)workspace;
  a.ml = (float*)((char*)workspace + al(pr * 128 * 4));
  a.out = out; a.fixed_ctx = ctx_len; a.block_len = block_len;
  a.active_chunks = nc;
  launch_attention_bf16(a, (hipStream_t)stream);
  return check_launch();
}

}  // namespace

// The allocation-free form's scratch: one array per GPU, in the library's
// device code object, holding the chunk partials of the last call.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in): its device address is looked up once per device with
// hipGetSymbolAddress and kept in g_scratch_dev.
static __device__ __align__(256) char scratch[ORTHRUS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];

int scratch_of_current_device(void** out) {
  int dev = -1;
  int rc = hip_ok(hipGetDevice(&dev));
  if (rc) return rc;
  if (dev < 0 || dev >= kMaxDevices) return ORTHRUS_EINVAL;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    rc = hip_ok(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (rc) return rc;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return ORTHRUS_OK;
}

}  // namespace

extern "C" {

int orthrus_block_attention(int32_t batch, int32_t rows, int32_t n_q_heads, int32_t n_kv_heads,
                            const void* q, const void* k_cache, const void* v_cache, int32_t cap,
                            int32_t ctx_len, const void* k_block, const void* v_block,
                            int32_t block_len, void* out, void* workspace,
                            uint64_t workspace_bytes, void* stream) {
  int rc = block_attention_args(batch, rows, n_q_heads, n_kv_heads, q, k_cache, v_cache, cap,
                                ctx_len, k_block, v_block, block_len, out);
  if (rc) return rc;
  if (!workspace) return ORTHRUS_EINVAL;
  uint64_t need = orthrus_attention_workspace(batch, rows, n_q_heads, n_kv_heads, ctx_len);
  if (workspace_bytes < need || !aligned(workspace)) return ORTHRUS_EINVAL;
  return block_attention_run(batch, rows, n_q_heads, n_kv_heads, q, k_cache, v_cache, cap,
                             ctx_len, k_block, v_block, block_len, out, workspace, stream);
}

int orthrus_block_attention_noalloc(int32_t batch, int32_t rows, int32_t n_q_heads,
                                    int32_t n_kv_heads, const void* q, const void* k_cache,
                                    const void* v_cache, int32_t cap, int32_t ctx_len,
                                    const void* k_block, const void* v_block, int32_t block_len,
                                    void* out, void* stream) {
  int rc = block_attention_args(batch, rows, n_q_heads, n_kv_heads, q, k_cache, v_cache, cap,
                                ctx_len, k_block, v_block, block_len, out);
  if (rc) return rc;
  if (orthrus_attention_workspace(batch, rows, n_q_heads, n_kv_heads, ctx_len) >
      ORTHRUS_NOALLOC_SCRATCH_BYTES)
    return ORTHRUS_ECAPACITY;
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc) return rc;
  return block_attention_run(batch, rows, n_q_heads, n_kv_heads, q, k_cache, v_cache, cap,
                             ctx_len, k_block, v_block, block_len, out, ws, stream);
}

int orthrus_stream_read(const void* buf, uint64_t bytes, uint32_t* out, int32_t n_workgroups,
                        void* stream) {
  if (!buf || !out || bytes == 0 || bytes % 16 || n_workgroups < 1 || !aligned(buf))
    return ORTHRUS_EINVAL;
  launch_stream_read(buf, bytes, out, n_workgroups, (hipStream_t)stream);
  return check_launch();
}

int32_t orthrus_default_attn_chunk(int32_t max_batch, int32_t max_ctx, int32_t n_kv_heads) {
  if (max_batch < 1 || max_ctx < 1 || n_kv_heads < 1) return ORTHRUS_EINVAL;
  return default_attn_chunk(max_batch, kv_slots(max_ctx), n_kv_heads);
}

const char* orthrus_strerror(int code) {
  switch (code) {
    case ORTHRUS_OK: return "ok";
    case ORTHRUS_EINVAL: return "invalid argument";
    case ORTHRUS_ECAPACITY: return "a sequence could grow past max_ctx";
    case ORTHRUS_ESTATE: return "call out of order";
    case ORTHRUS_EHIP: return "HIP error";
  }
  return "unknown error";
}

int orthrus_last_hip_error(void) { return g_last_hip; }

}  // extern "C"
