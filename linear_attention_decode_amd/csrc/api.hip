// C ABI of the KDA library (include/kda.h): validation, workspace layout, launch
// sequencing per layer, hipGraph capture of the decode step, and event timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kda.h"
#include "kda_internal.h"
#include "skinny.h"

using namespace kda;

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

#define KDA_HIP(call)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(KDA_E_HIP, "%s failed: %s", #call, hipGetErrorString(e_));           \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

struct LayerDev {
  PackedMat wq, wk, wv, wo, fa, fb, wbeta, ga, gb;
  const float* conv_w;
  const float* a_log;
  const float* dt_bias;
  const float* o_norm_w;
  // The model's own copy of the Q8_0 weights in matrix-core order (made for one-launch
  // eligible stacks; null otherwise): the fused projection rows and W_o (bytes and scales),
  // F_b and G_b in gate-tile order.  Where it exists every kernel reads it and never the
  // caller's packed buffers.
  const int8_t* pw = nullptr;
  const uint16_t* pd = nullptr;
  const int8_t* ow = nullptr;
  const uint16_t* od = nullptr;
  const int8_t* fbw = nullptr;
  const uint16_t* fbd = nullptr;
  const int8_t* gbw = nullptr;
  const uint16_t* gbd = nullptr;
};

// A captured hipGraph of one op (decode, verify or commit) and the arguments it was
// captured for (pointers, sizes, stream): replayed while they match, captured again when
// one changes.
struct GraphSlot {
  std::vector<uintptr_t> key;
  hipGraphExec_t exec = nullptr;
};
enum { kGraphDecode = 0, kGraphVerify = 1, kGraphVerifyOdd = 2, kGraphCommit = 3, kGraphSlots = 4 };

// A verify log on one state: which half of the log the last verify wrote (and for how many
// tokens) while no commit of it is recorded, and the half and length of a commit recorded
// by kda_verify_commit and not yet applied to the state (-1: none).
struct LogRec {
  const float* S = nullptr;
  const float* conv = nullptr;
  int B = 0;
  const void* log = nullptr;
  size_t log_bytes = 0;
  int last_half = -1, last_T = 0;
  int pend_half = -1, pend_T = 0;
};

struct TimedLaunch {
  hipEvent_t a, b;
  int kind;
};

struct kda_model {
  kda_dims d;
  std::vector<LayerDev> layers;
  int C = 0, Kq = 0, V = 0, proj_rows = 0, proj_stride = 0;
  float q_scale = 0.f;
  // options
  bool use_graph = false;
  bool timing = false;
  // graph cache (decode, verify, commit)
  hipStream_t cap_stream = nullptr;
  GraphSlot graphs[kGraphSlots];
  // verify logs in use on this model's states (the folded commit's bookkeeping)
  std::vector<LogRec> logs;
  // one-launch decode (batch 1)
  bool use_persist = true;
  bool coop = false;                // cooperative launch of the one-launch decode
  bool pers_ok = false;
  int pers_blocks = 0;
  int wall_khz = 0;                 // wall-clock ticks per millisecond
  PersistLayer* d_layers = nullptr;
  int8_t* mma_w = nullptr;          // projection rows and W_o of every layer, matrix-core order
  float* dtb_rep = nullptr;         // scalar-gate stack: dt_bias[h] repeated over the head's d_k
  uint64_t* xchg = nullptr;         // exchange words (xbuf | pbuf | gbuf | obuf)
  int* err = nullptr;
  int* err_host = nullptr;          // host-mapped: set by a step whose wait between blocks ran out
  uint32_t epoch = 0;
  PersistParams pp;
  // timing
  std::vector<TimedLaunch> pool;
  size_t used = 0;
  double total_ms[KDA_K_COUNT] = {0};
  int64_t count[KDA_K_COUNT] = {0};
};

// ---------------------------------------------------------------------------------------
// Workspace layout (decode / verify): proj [N][proj_stride] | alpha,gate [N][K+V] |
// o [N][V] | gate [N][V] | ss [N][H][V/kHeadCols]; each region 256-byte aligned.
// Verify log per layer: proj rows [N][proj_stride] then alpha,gate [N][K+V].
// ---------------------------------------------------------------------------------------
namespace {

struct WsLayout {
  size_t proj = 0, ag = 0, o = 0, gate = 0, ss = 0, sk = 0, total = 0;
};

WsLayout ws_layout(const kda_model* m, int64_t N) {
  WsLayout w;
  size_t off = 0;
  w.proj = off; off = align_up(off + (size_t)N * m->proj_stride * 4, 256);
  w.ag = off;   off = align_up(off + (size_t)N * (m->Kq + m->V) * 4, 256);
  w.o = off;    off = align_up(off + (size_t)N * m->V * 4, 256);
  w.gate = off; off = align_up(off + (size_t)N * m->V * 4, 256);
  w.ss = off;   off = align_up(off + (size_t)N * m->d.n_heads * (m->d.d_v / kHeadCols) * 4, 256);
  // MFMA column-fragment scratch of the skinny projections (Q8_0 with 9..64 columns, or
  // 1..64 for a model with its own matrix-core copy)
  const int Kmax = std::max(m->d.d_model, m->V);
  w.sk = off;
  if (m->mma_w) off = align_up(off + skinny_scratch_bytes((int)std::min<int64_t>(N, 64), Kmax), 256);
  else if (skinny_supported(m->d.wtype, (int)N, m->d.d_model) || skinny_supported(m->d.wtype, (int)N, m->V))
    off = align_up(off + skinny_scratch_bytes((int)N, Kmax), 256);
  w.total = off;
  return w;
}

// Workspace layout (prefill, M = B*L tokens, NC = B*H*nch chunks).
struct PfLayout {
  size_t P = 0, xs = 0, W = 0, U = 0, Qt = 0, Kt = 0, A = 0, dec = 0, o = 0, on = 0, total = 0;
};

PfLayout pf_layout(const kda_model* m, int64_t B, int64_t L) {
  const kda_dims& d = m->d;
  const int64_t M = B * L, nch = (L + kChunk - 1) / kChunk, NC = B * d.n_heads * nch;
  const int64_t K = m->Kq, V = m->V;
  PfLayout w;
  size_t off = 0;
  auto take = [&](size_t& dst, int64_t floats) { dst = off; off = align_up(off + (size_t)floats * 4, 256); };
  take(w.P, M * m->proj_stride);
  take(w.xs, M * d.d_model);          // fp32 x as two BF16 planes (F32 input only)
  take(w.W, NC * kChunk * d.d_k);
  take(w.U, NC * kChunk * d.d_v);
  take(w.Qt, NC * kChunk * d.d_k);
  take(w.Kt, NC * kChunk * d.d_k);
  take(w.A, NC * kChunk * kChunk);
  take(w.dec, NC * d.d_k);
  take(w.o, M * V);
  take(w.on, M * V);                  // gated norm as two BF16 planes
  w.total = off;
  return w;
}

int flush_timing(kda_model* m) {
  for (size_t i = 0; i < m->used; ++i) {
    TimedLaunch& t = m->pool[i];
    KDA_HIP(hipEventSynchronize(t.b));
    float ms = 0.f;
    KDA_HIP(hipEventElapsedTime(&ms, t.a, t.b));
    m->total_ms[t.kind] += ms;
    m->count[t.kind] += 1;
  }
  m->used = 0;
  return KDA_OK;
}

// Launch wrapper: optional event pair around the launch.
template <typename F>
int timed(kda_model* m, int kind, hipStream_t s, bool record, F&& launch) {
  TimedLaunch* t = nullptr;
  if (record) {
    if (m->used >= 65536) {
      int r = flush_timing(m);
      if (r != KDA_OK) return r;
    }
    if (m->used == m->pool.size()) {
      TimedLaunch n{};
      n.kind = kind;
      KDA_HIP(hipEventCreate(&n.a));
      KDA_HIP(hipEventCreate(&n.b));
      m->pool.push_back(n);
    }
    t = &m->pool[m->used++];
    t->kind = kind;
    KDA_HIP(hipEventRecord(t->a, s));
  }
  hipError_t e = launch();
  if (e != hipSuccess) return fail(KDA_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  if (record) KDA_HIP(hipEventRecord(t->b, s));
  return KDA_OK;
}

// Segment table of the fused input projection: q | k | v | f_a | g_a | beta.
void proj_segments(const kda_model* m, const LayerDev& L, GemvParams& p, bool conv) {
  const kda_dims& d = m->d;
  const PackedMat mats[6] = {L.wq, L.wk, L.wv, L.fa, L.ga, L.wbeta};
  const int rows[6] = {m->Kq, m->Kq, m->V, d.rank_f, d.rank_g, d.n_heads};
  int tile = 0, off = 0;
  for (int i = 0; i < 6; ++i) {
    GemvSeg& s = p.seg[i];
    s.m = mats[i];
    if (L.pw) {
      // the model's copy: each matrix starts at a 16-row tile of the fused rows
      s.m = PackedMat{};
      s.m.w = reinterpret_cast<const uint8_t*>(L.pw) + (size_t)off * d.d_model;
      s.m.d = reinterpret_cast<const __half*>(L.pd) + (size_t)off * (d.d_model / 32);
    }
    s.rows = rows[i];
    s.first_tile = tile;
    s.out_off = off;
    s.conv_chan = (conv && i < 3) ? off : -1;
    tile += (rows[i] + kGemvRowsPerBlock - 1) / kGemvRowsPerBlock;
    off += rows[i];
  }
  p.nseg = 6;
  p.mma = L.pw ? 1 : 0;
}

int proj_grid(const GemvParams& p) {
  const GemvSeg& s = p.seg[p.nseg - 1];
  return s.first_tile + (s.rows + kGemvRowsPerBlock - 1) / kGemvRowsPerBlock;
}

int enqueue_gates(kda_model* m, const LayerDev& L, const float* proj, int N, float* ag,
                  hipStream_t s, bool rec) {
  const kda_dims& d = m->d;
  GatesParams gp;
  gp.N = N; gp.K = m->Kq; gp.V = m->V; gp.dk = d.d_k; gp.rank = d.rank_f; gp.C = m->C;
  gp.wt = d.wtype; gp.proj = proj; gp.proj_stride = m->proj_stride;
  gp.fb = L.fb; gp.gb = L.gb; gp.a_log = L.a_log; gp.dt_bias = L.dt_bias; gp.out = ag;
  gp.gate = d.gate; gp.gate_lb = d.gate_lb;
  gp.fbw = L.fbw; gp.fbd = L.fbd; gp.gbw = L.gbw; gp.gbd = L.gbd;
  return timed(m, KDA_K_GATES, s, rec, [&] { return launch_gates(gp, s); });
}

// A matrix-core product over any number of columns, for a model with its own weight copy:
// launches of at most 64 columns (whole sequences of T tokens each when the verify conv
// runs in the epilogue), every per-column pointer moved on by the launch's first column.
hipError_t launch_skinny_cols(int prologue, const GemvParams& g, int T, void* scratch, hipStream_t s) {
  const int per = g.act ? (64 / T) * T : 64;
  for (int n0 = 0; n0 < g.N; n0 += per) {
    GemvParams c = g;
    c.N = std::min(per, g.N - n0);
    if (c.x) c.x += (size_t)n0 * g.x_stride;
    if (c.o) c.o += (size_t)n0 * g.K;
    if (c.gate) c.gate += (size_t)n0 * g.K;
    if (c.ss) c.ss += (size_t)n0 * g.H * g.ncb;
    c.out += (size_t)n0 * g.out_stride;
    if (c.resid) c.resid += (size_t)n0 * g.out_stride;
    if (c.act) {
      const int b0 = n0 / T;
      c.act += (size_t)n0 * g.C;
      if (c.win) c.win += (size_t)b0 * 3 * g.C;
      if (c.pre_proj) c.pre_proj += (size_t)b0 * g.pre_T * g.out_stride;
      if (c.pre_ntok) c.pre_ntok += b0;
    } else {
      if (c.win) c.win += (size_t)n0 * 3 * g.C;
      if (c.active) c.active += n0;
    }
    const hipError_t e = launch_skinny(prologue, c, scratch, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// One layer of decode (T = 1) or verify (T > 1): projections, gates, per-head step, o_proj.
// Verify passes `act`: the projections stay pre-conv (they are logged for the commit's
// window roll) and the activated q|k|v go to act; decode applies the conv in the
// projection epilogue and rolls the window there.
// The previous verify's log rows of one layer, replayed ahead of this verify's tokens (a
// commit folded into the verify after it).
struct FoldSrc {
  const float* proj = nullptr;
  const float* ag = nullptr;
  const float* act = nullptr;
  const int* ntok = nullptr;      // accepted tokens per sequence (the log header)
  int T = 0;                      // tokens per sequence of that verify
};

int enqueue_layer(kda_model* m, int l, const float* x_in, float* y, int B, int T,
                  float* S, float* win, float* proj, float* ag, float* act, const WsLayout& wl,
                  char* ws, bool write_state, hipStream_t s, bool rec,
                  const int* active = nullptr, bool roll = false, const FoldSrc* fold = nullptr) {
  const kda_dims& d = m->d;
  const LayerDev& L = m->layers[l];
  const int N = B * T;
  const bool decode = (T == 1) && write_state && !act;   // (the scan passes act: conv apart)
  float* o = reinterpret_cast<float*>(ws + wl.o);
  float* gate = reinterpret_cast<float*>(ws + wl.gate);
  float* ss = reinterpret_cast<float*>(ws + wl.ss);

  // the matrix-core products: always for a model with its own weight copy (which only they
  // read), else for 9..64 columns; verify there runs its conv in the projection epilogue
  const bool mma = L.pw != nullptr;
  auto use_skinny = [&](int K) { return mma || skinny_supported(d.wtype, N, K); };
  const bool conv_fused = act && use_skinny(d.d_model);
  GemvParams pp;
  proj_segments(m, L, pp, decode || conv_fused);
  pp.K = d.d_model;
  pp.N = N;
  pp.wt = d.wtype;
  pp.x = x_in;
  pp.x_stride = d.d_model;
  pp.prenorm = d.prenorm_residual;
  pp.eps = d.norm_eps;
  pp.out = proj;
  pp.out_stride = m->proj_stride;
  pp.conv_w = L.conv_w;
  pp.win = win;
  pp.C = m->C;
  pp.active = active;
  if (conv_fused) {
    pp.act = act;
    pp.T = T;
  }
  if (fold) {
    pp.pre_proj = fold->proj;
    pp.pre_ntok = fold->ntok;
    pp.pre_T = fold->T;
  }
  const int g1 = proj_grid(pp);
  int r = timed(m, KDA_K_PROJ, s, rec, [&] {
    if (mma) return launch_skinny_cols(kProX, pp, T, ws + wl.sk, s);
    if (use_skinny(pp.K)) return launch_skinny(kProX, pp, ws + wl.sk, s);
    return launch_gemv(d.wtype, kProX, pp, g1, s);
  });
  if (r) return r;

  if (act && !conv_fused) {
    r = timed(m, KDA_K_PROJ, s, rec, [&] {
      return launch_conv_seq(proj, m->proj_stride, win, L.conv_w, act, B, T, m->C,
                             fold ? fold->proj : nullptr, fold ? fold->ntok : nullptr,
                             fold ? fold->T : 0, s);
    });
    if (r) return r;
  }
  // one token a sequence for a few sequences: the head kernel computes its own gates (each
  // of its waves re-reads all of its head's F_b rows, which a wide batch would pay for); a
  // model with its own gate-tile-order copy on the matrix cores, others with vector dots.
  // (A matrix-core form for up to 8 tokens cost more than the separate launch at verify's 4
  // tokens a sequence: 22.8 us against 11.3 + 7.1.)
  const bool mfma_gates = L.fbw && d.gate == KDA_GATE_KDA && d.d_k == 128 &&
                          (d.rank_f == 32 || d.rank_f == 64 || d.rank_f == 128) && T == 1 &&
                          !fold && B <= kFuseGatesMaxBOwned;
  const bool fuse_gates = mfma_gates || (decode && !fold && !L.fbw && B <= kFuseGatesMaxB);
  if (!fuse_gates) {
    r = enqueue_gates(m, L, proj, N, ag, s, rec);
    if (r) return r;
  }

  HeadParams hp;
  hp.H = d.n_heads; hp.dk = d.d_k; hp.dv = d.d_v; hp.C = m->C;
  hp.rank_f = d.rank_f; hp.rank_g = d.rank_g;
  hp.B = B; hp.T = T;
  hp.proj = proj; hp.proj_stride = m->proj_stride;
  hp.act = act;
  hp.wt = d.wtype; hp.fb = L.fb; hp.gb = L.gb;
  hp.a_log = L.a_log; hp.dt_bias = L.dt_bias;
  hp.alpha_gate = ag;
  hp.S = S; hp.write_state = write_state ? 1 : 0;
  hp.ntok = nullptr; hp.write_out = 1;
  hp.o = o; hp.gate = gate; hp.ss = ss;
  hp.l2_eps = d.l2_eps; hp.q_scale = m->q_scale;
  hp.active = active;
  // a multi-token step that keeps its state (the sequential-scan prefill) rolls the window
  // by all T tokens after the state write, in the same launch
  if (roll) hp.win_commit = win;
  if (fuse_gates) {
    hp.fuse_gates = mfma_gates ? 2 : 1;
    if (act) hp.ag_out = ag;       // verify and scan: a replay of these tokens reads them
    hp.gate_form = d.gate; hp.gate_lb = d.gate_lb;
    hp.fbw = L.fbw; hp.fbd = L.fbd; hp.gbw = L.gbw; hp.gbd = L.gbd;
  }
  if (fold) {
    hp.pre_proj = fold->proj;
    hp.pre_act = fold->act;
    hp.pre_ag = fold->ag;
    hp.pre_ntok = fold->ntok;
    hp.pre_T = fold->T;
  }
  r = timed(m, KDA_K_HEAD, s, rec, [&] { return launch_head(hp, s); });
  if (r) return r;

  GemvParams po;
  po.seg[0].m = L.wo;
  if (mma) {
    po.seg[0].m = PackedMat{};
    po.seg[0].m.w = reinterpret_cast<const uint8_t*>(L.ow);
    po.seg[0].m.d = reinterpret_cast<const __half*>(L.od);
    po.mma = 1;
  }
  po.seg[0].rows = d.d_model;
  po.seg[0].first_tile = 0;
  po.seg[0].out_off = 0;
  po.seg[0].conv_chan = -1;
  po.nseg = 1;
  po.K = m->V;
  po.N = N;
  po.wt = d.wtype;
  po.o = o; po.gate = gate; po.ss = ss; po.onw = L.o_norm_w;
  po.H = d.n_heads; po.dv = d.d_v; po.ncb = d.d_v / kHeadCols;
  po.eps = d.norm_eps;
  po.out = y;
  po.out_stride = d.d_model;
  po.resid = d.prenorm_residual ? x_in : nullptr;
  const int g2 = (d.d_model + kGemvRowsPerBlock - 1) / kGemvRowsPerBlock;
  return timed(m, KDA_K_OUT, s, rec, [&] {
    if (mma) return launch_skinny_cols(kProGatedNorm, po, T, ws + wl.sk, s);
    if (use_skinny(po.K)) return launch_skinny(kProGatedNorm, po, ws + wl.sk, s);
    return launch_gemv(d.wtype, kProGatedNorm, po, g2, s);
  });
}

size_t state_layer_stride(const kda_model* m, int B) {
  return (size_t)B * m->d.n_heads * m->d.d_k * m->d.d_v;
}
size_t win_layer_stride(const kda_model* m, int B) { return (size_t)B * (m->d.conv_k - 1) * m->C; }

int enqueue_decode(kda_model* m, const float* x, float* y, const kda_state* st, char* ws,
                   hipStream_t s, bool rec, const int* active = nullptr) {
  const int B = st->batch;
  WsLayout wl = ws_layout(m, B);
  float* proj = reinterpret_cast<float*>(ws + wl.proj);
  float* ag = reinterpret_cast<float*>(ws + wl.ag);
  for (int l = 0; l < m->d.n_layers; ++l) {
    const float* xin = (l == 0 || !m->d.prenorm_residual) ? x : y;
    int r = enqueue_layer(m, l, xin, y, B, 1, st->S_dev + l * state_layer_stride(m, B),
                          st->conv_dev + l * win_layer_stride(m, B), proj, ag, nullptr, wl, ws,
                          true, s, rec, active);
    if (r) return r;
  }
  return KDA_OK;
}

void drop_graph(kda_model* m) {
  for (GraphSlot& g : m->graphs) {
    if (g.exec) (void)hipGraphExecDestroy(g.exec);
    g.exec = nullptr;
    g.key.clear();
  }
}

// Replays the op's graph for `key`, capturing `enqueue` (on the model's capture stream)
// first when the slot holds none or one for other arguments.
template <typename F>
int run_graph(kda_model* m, int slot, std::vector<uintptr_t> key, hipStream_t s, F&& enqueue) {
  GraphSlot& g = m->graphs[slot];
  key.push_back((uintptr_t)s);
  if (!g.exec || g.key != key) {
    if (g.exec) (void)hipGraphExecDestroy(g.exec);
    g.exec = nullptr;
    g.key.clear();
    hipGraph_t graph = nullptr;
    KDA_HIP(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeRelaxed));
    const int r = enqueue(m->cap_stream);
    hipError_t e = hipStreamEndCapture(m->cap_stream, &graph);
    if (r) { if (graph) (void)hipGraphDestroy(graph); return r; }
    if (e != hipSuccess) return fail(KDA_E_HIP, "graph capture: %s", hipGetErrorString(e));
    e = hipGraphInstantiate(&g.exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) { g.exec = nullptr; return fail(KDA_E_HIP, "graph instantiate: %s", hipGetErrorString(e)); }
    g.key = std::move(key);
  }
  KDA_HIP(hipGraphLaunch(g.exec, s));
  return KDA_OK;
}

int check_state(const kda_model* m, const kda_state* st) {
  if (!st || !st->S_dev || !st->conv_dev) return fail(KDA_E_ARG, "null state");
  if (st->batch < 1) return fail(KDA_E_SHAPE, "state batch %d < 1", st->batch);
  if (!aligned16(st->S_dev) || !aligned16(st->conv_dev)) return fail(KDA_E_ALIGN, "state not 16-byte aligned");
  return KDA_OK;
}

// ---- verify logs: a header of the accepted lengths ([B] int32, 256-byte aligned), then two
// halves that alternate between consecutive verifies (the one being written, the one whose
// commit it folds in).  A half holds per layer: pre-conv projections [B T][proj_stride] |
// alpha, gate [B T][K + V] | activated q|k|v [B T][C].
size_t log_hdr_bytes(int B) { return align_up((size_t)B * 4, 256); }
size_t log_layer_floats(const kda_model* m, int B, int T) {
  return (size_t)B * T * (m->proj_stride + m->Kq + m->V + m->C);
}
size_t log_half_bytes(const kda_model* m, int B, int T) {
  return align_up(log_layer_floats(m, B, T) * m->d.n_layers * 4, 256);
}
size_t log_half_cap(size_t log_bytes, int B) {
  const size_t hdr = log_hdr_bytes(B);
  return log_bytes < hdr ? 0 : ((log_bytes - hdr) / 2) & ~size_t(255);
}

struct LogLayer {
  float* proj;
  float* ag;
  float* act;
};
LogLayer log_layer(const kda_model* m, const void* log, size_t log_bytes, int B, int T, int half,
                   int l) {
  char* base = static_cast<char*>(const_cast<void*>(log)) + log_hdr_bytes(B) +
               (size_t)half * log_half_cap(log_bytes, B);
  float* lp = reinterpret_cast<float*>(base) + (size_t)l * log_layer_floats(m, B, T);
  LogLayer r;
  r.proj = lp;
  r.ag = lp + (size_t)B * T * m->proj_stride;
  r.act = r.ag + (size_t)B * T * (m->Kq + m->V);
  return r;
}

bool same_state(const LogRec& r, const kda_state* st) {
  return r.S == st->S_dev || r.conv == st->conv_dev;
}

LogRec* find_log(kda_model* m, const kda_state* st, const void* log, size_t log_bytes) {
  for (auto& r : m->logs)
    if (r.S == st->S_dev && r.conv == st->conv_dev && r.B == st->batch && r.log == log &&
        r.log_bytes == log_bytes)
      return &r;
  return nullptr;
}

// Apply a recorded commit: each layer's head kernel replays the accepted tokens from the log
// into the state, then rolls the window by their logged pre-conv projections.
int apply_commit(kda_model* m, LogRec& rc, hipStream_t s, bool eager) {
  const kda_dims& d = m->d;
  const int B = rc.B, T = rc.pend_T, half = rc.pend_half;
  const int* accept = static_cast<const int*>(rc.log);
  float* S = const_cast<float*>(rc.S);
  float* conv = const_cast<float*>(rc.conv);
  auto enqueue = [&](hipStream_t cs, bool rec) {
    for (int l = 0; l < d.n_layers; ++l) {
      const LayerDev& L = m->layers[l];
      const LogLayer ll = log_layer(m, rc.log, rc.log_bytes, B, T, half, l);
      HeadParams hp;
      hp.H = d.n_heads; hp.dk = d.d_k; hp.dv = d.d_v; hp.C = m->C;
      hp.rank_f = d.rank_f; hp.rank_g = d.rank_g;
      hp.B = B; hp.T = T;
      hp.proj = ll.proj; hp.proj_stride = m->proj_stride;
      hp.act = ll.act;
      hp.alpha_gate = ll.ag;
      hp.wt = d.wtype; hp.fb = L.fb; hp.gb = L.gb;
      hp.a_log = L.a_log; hp.dt_bias = L.dt_bias;
      hp.S = S + (size_t)l * B * d.n_heads * d.d_k * d.d_v;
      hp.write_state = 1; hp.ntok = accept; hp.write_out = 0;
      hp.l2_eps = d.l2_eps; hp.q_scale = m->q_scale;
      // the window roll runs in the same launch, after the replay
      hp.win_commit = conv + (size_t)l * B * (d.conv_k - 1) * m->C;
      const int rr = timed(m, KDA_K_COMMIT, cs, rec, [&] { return launch_head(hp, cs); });
      if (rr) return rr;
    }
    return (int)KDA_OK;
  };
  int r;
  if (!m->use_graph || m->timing || eager) {
    r = enqueue(s, m->timing && !eager);
  } else {
    const std::vector<uintptr_t> key = {(uintptr_t)rc.S, (uintptr_t)rc.conv, (uintptr_t)rc.log,
                                        (uintptr_t)rc.log_bytes, (uintptr_t)B, (uintptr_t)T,
                                        (uintptr_t)half};
    r = run_graph(m, kGraphCommit, key, s, [&](hipStream_t cs) { return enqueue(cs, false); });
  }
  rc.pend_half = -1;
  return r;
}

// Before a call that reads or writes a state: apply the commits pending on it (except the
// one `keep` folds in itself; `eager`: launched directly, no graph captured).  A call that
// writes the state (`writes`) also retires every verify on it not yet committed: a commit
// after it would no longer follow its verify.
int flush_state(kda_model* m, const kda_state* st, hipStream_t s, bool writes,
                const LogRec* keep = nullptr, bool eager = false) {
  for (auto& rc : m->logs) {
    if (&rc == keep || !same_state(rc, st)) continue;
    if (rc.pend_half >= 0) {
      const int r = apply_commit(m, rc, s, eager);
      if (r) return r;
    }
    if (writes) rc.last_half = -1;
  }
  return KDA_OK;
}

// Before a verify writes `log`: a commit pending through the same memory for another state
// is applied first (its rows are about to be overwritten), and that state's uncommitted
// verify through it is retired.
int flush_log(kda_model* m, const void* log, const kda_state* st, hipStream_t s) {
  for (auto& rc : m->logs) {
    if (rc.log != log || same_state(rc, st)) continue;
    if (rc.pend_half >= 0) {
      const int r = apply_commit(m, rc, s, false);
      if (r) return r;
    }
    rc.last_half = -1;
  }
  return KDA_OK;
}

// The record of (state, log), made if there is none; records with nothing left to commit or
// apply are dropped first.  At most kMaxLogs verifies wait for a commit at once (the oldest
// is retired beyond that); null if that many commits are pending.
constexpr size_t kMaxLogs = 64;
LogRec* add_log(kda_model* m, const kda_state* st, const void* log, size_t log_bytes) {
  if (LogRec* r = find_log(m, st, log, log_bytes)) return r;
  m->logs.erase(std::remove_if(m->logs.begin(), m->logs.end(),
                               [](const LogRec& rc) { return rc.last_half < 0 && rc.pend_half < 0; }),
                m->logs.end());
  if (m->logs.size() >= kMaxLogs) {
    auto it = std::find_if(m->logs.begin(), m->logs.end(),
                           [](const LogRec& rc) { return rc.pend_half < 0; });
    if (it == m->logs.end()) return nullptr;
    m->logs.erase(it);
  }
  LogRec rc;
  rc.S = st->S_dev;
  rc.conv = st->conv_dev;
  rc.B = st->batch;
  rc.log = log;
  rc.log_bytes = log_bytes;
  m->logs.push_back(rc);
  return &m->logs.back();
}

// One-launch decode: eligible for batch 1, Q8_0 (or MXFP4, held for it as the exactly equal
// Q8_0) stacks with the KDA gate, the lower-bounded one or the scalar one (whose per-head
// F_b row and dt_bias it takes repeated over the head's channels), d_k = d_v = 128, H*d_v = D in
// {1024, 2048}, low-rank gates of rank 32, 64 or 128, and enough co-resident blocks for the
// static work split (two blocks per head, D/16 output-projection blocks after them, at most
// 32 projection rows per remaining block).
size_t exchange_words(const kda_model* m) {
  return 2 * (size_t)m->d.d_model + m->proj_rows + m->V + 8 * (size_t)m->d.n_heads +
         3 * (size_t)kMaxPersistBlocks;
}

// The bound of every wait between blocks of the one-launch decode: `us` microseconds of wall
// clock, or 50 ms when us <= 0.  Under 100 us the flag waits look at the clock after every
// poll round (a limit that short is for exercising the timeout path).
void set_wait_limit(kda_model* m, int64_t us) {
  PersistParams& p = m->pp;
  if (us <= 0) {
    p.timeout = (uint64_t)m->wall_khz * 50;
    p.poll_rounds = 48;
  } else {
    p.timeout = std::max<uint64_t>(1, (uint64_t)m->wall_khz * (uint64_t)us / 1000);
    p.poll_rounds = us < 100 ? 1 : 48;
  }
}

hipError_t persist_setup(kda_model* m, const kda_layer* layers) {
  const kda_dims& d = m->d;
  const int nb = persistent_max_blocks();
  const int ob0 = 2 * d.n_heads, nob = d.d_model / 32;
  const int rank = d.rank_f;
  const bool mx4 = d.wtype == KDA_MXFP4, scal = d.gate == KDA_GATE_SCALAR;
  const bool safe = d.gate == KDA_GATE_SAFE;
  bool ok = nb > 0 && nb <= kMaxPersistBlocks && (d.wtype == KDA_Q8_0 || mx4) && d.prenorm_residual &&
            (d.gate == KDA_GATE_KDA || scal || safe) &&
            d.d_k == 128 && d.d_v == 128 && m->V == d.d_model &&
            (d.d_model == 1024 || d.d_model == 2048) && d.rank_f == d.rank_g &&
            (rank == 32 || rank == 64 || rank == 128);
  if (ok) {
    // heads, output bands of 32 rows, q/k/v rows 48 per block, low-rank and beta rows 16 per
    // block
    const int nq = m->C / 48, nl = (m->proj_rows - m->C + 15) / 16;
    ok = d.n_heads <= 32 && m->C % 48 == 0 && ob0 + nob + nq + nl <= nb;
  }
  if (!ok) return hipSuccess;
  // the rows the kernel streams, rearranged once for the matrix cores
  const int D = d.d_model;
  const size_t pw = mma_order_bytes(m->proj_rows, D), pd = mma_order_scales(m->proj_rows, D);
  const size_t ow = mma_order_bytes(D, D), od = mma_order_scales(D, D);
  const int KF = d.n_heads * d.d_k, KG = m->V, nbr = rank / 32;
  const size_t per_layer = pw + ow + 2 * (pd + od) + (size_t)(KF + KG) * (rank + 2 * nbr);
  hipError_t e = hipMalloc(&m->mma_w, per_layer * d.n_layers);
  if (e != hipSuccess) return e;
  // MXFP4: a layer's matrices are first expanded to the Q8_0 layout holding the same values
  // (twice each E2M1 value as the int8 code, half the E8M0 scale as the fp16 one), in a
  // scratch area reused layer by layer; the scalar gate's F_b (one row a head) is repeated
  // there over the head's d_k rows.  The per-layer kernels of such a stack keep reading the
  // caller's buffers; only the one-launch kernel reads the copy.
  const int FR = scal ? d.n_heads : KF;          // F_b rows as the caller packed them
  const int64_t xr[10] = {m->Kq, m->Kq, m->V, d.rank_f, d.rank_g, d.n_heads, D, FR, KG, KF};
  const int64_t xc[10] = {D, D, D, D, D, D, m->V, rank, rank, rank};
  size_t xoff[11] = {};
  uint8_t* xq = nullptr;
  int* xbad = nullptr;
  if (mx4 || scal) {
    for (int i = 0; i < 10; ++i) {
      const bool used = i < 9 ? mx4 : scal;
      xoff[i + 1] = xoff[i] + (used ? align_up(q8_scale_offset(xr[i], xc[i]) + (size_t)xr[i] * (xc[i] / 32) * 2, 256) : 0);
    }
    e = hipMalloc(&xq, xoff[10]);
    if (e == hipSuccess) e = hipMalloc(&xbad, sizeof(int));
    if (e == hipSuccess) e = hipMemset(xbad, 0, sizeof(int));
    if (e == hipSuccess && scal) e = hipMalloc(&m->dtb_rep, sizeof(float) * KF * d.n_layers);
  }
  std::vector<PersistLayer> host(d.n_layers);
  for (int l = 0; l < d.n_layers && e == hipSuccess; ++l) {
    const LayerDev& L = m->layers[l];
    PersistLayer& P = host[l];
    P.seg[0] = L.wq; P.seg[1] = L.wk; P.seg[2] = L.wv; P.seg[3] = L.fa; P.seg[4] = L.ga; P.seg[5] = L.wbeta;
    P.wo = L.wo;
    P.conv_w = L.conv_w; P.a_log = L.a_log; P.dt_bias = L.dt_bias; P.o_norm_w = L.o_norm_w;
    int8_t* base = m->mma_w + per_layer * l;
    P.pw = base;
    P.ow = base + pw;
    P.pd = reinterpret_cast<const uint16_t*>(base + pw + ow);
    P.od = P.pd + pd;
    int8_t* gbase = base + pw + ow + 2 * (pd + od);
    P.fbw = gbase;
    P.gbw = gbase + (size_t)KF * rank;
    P.fbd = reinterpret_cast<const uint16_t*>(gbase + (size_t)(KF + KG) * rank);
    P.gbd = P.fbd + (size_t)KF * nbr;
    // the Q8_0 sources: the caller's matrices, or their expansion (W_q, W_k, W_v, F_a, G_a,
    // W_beta, W_o, F_b, G_b)
    PackedMat q8[9] = {L.wq, L.wk, L.wv, L.fa, L.ga, L.wbeta, L.wo, L.fb, L.gb};
    if (mx4) {
      for (int i = 0; i < 9 && e == hipSuccess; ++i) {
        e = launch_mx4_to_q8(q8[i].w, xr[i], xc[i], xq + xoff[i], xbad, nullptr);
        q8[i] = packed_view(xq + xoff[i], kQ8, xr[i], xc[i]);
      }
      if (e != hipSuccess) break;
    }
    if (scal) {
      e = launch_q8_repeat_rows(q8[7].w, d.n_heads, rank, d.d_k, xq + xoff[9], nullptr);
      q8[7] = packed_view(xq + xoff[9], kQ8, KF, rank);
      if (e == hipSuccess)
        e = launch_f32_repeat(L.dt_bias, d.n_heads, d.d_k, m->dtb_rep + (size_t)l * KF, nullptr);
      P.dt_bias = m->dtb_rep + (size_t)l * KF;
      if (e != hipSuccess) break;
    }
    const int rows[6] = {m->Kq, m->Kq, m->V, d.rank_f, d.rank_g, d.n_heads};
    MmaSource src{};
    int first = 0;
    for (int i = 0; i < 6; ++i) {
      src.w[i] = q8[i].w;
      src.d[i] = q8[i].d;
      src.first[i] = first;
      first += rows[i];
    }
    src.nseg = 6;
    e = launch_mma_order(src, m->proj_rows, D, const_cast<int8_t*>(P.pw), const_cast<uint16_t*>(P.pd), nullptr);
    if (e != hipSuccess) break;
    MmaSource so{};
    so.w[0] = q8[6].w;
    so.d[0] = q8[6].d;
    so.nseg = 1;
    e = launch_mma_order(so, D, D, const_cast<int8_t*>(P.ow), const_cast<uint16_t*>(P.od), nullptr);
    if (e != hipSuccess) break;
    e = launch_gate_order(q8[7].w, q8[7].d, KF, rank, const_cast<int8_t*>(P.fbw), const_cast<uint16_t*>(P.fbd), nullptr);
    if (e != hipSuccess) break;
    e = launch_gate_order(q8[8].w, q8[8].d, KG, rank, const_cast<int8_t*>(P.gbw), const_cast<uint16_t*>(P.gbd), nullptr);
    // (the scratch is rewritten by the next layer's expansion)
    if ((mx4 || scal) && e == hipSuccess) e = hipDeviceSynchronize();
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  int bad = 0;
  if (mx4 && e == hipSuccess && xbad) e = hipMemcpy(&bad, xbad, sizeof(int), hipMemcpyDeviceToHost);
  if (xq) (void)hipFree(xq);
  if (xbad) (void)hipFree(xbad);
  if (e != hipSuccess) return e;
  if (bad) {
    // a scale with no fp16 power of two: the stack stays on the per-layer kernels
    (void)hipFree(m->mma_w);
    m->mma_w = nullptr;
    if (m->dtb_rep) (void)hipFree(m->dtb_rep);
    m->dtb_rep = nullptr;
    return hipSuccess;
  }
  (void)layers;
  e = hipMalloc(&m->d_layers, sizeof(PersistLayer) * d.n_layers);
  if (e != hipSuccess) return e;
  e = hipMemcpy(m->d_layers, host.data(), sizeof(PersistLayer) * d.n_layers, hipMemcpyHostToDevice);
  if (e != hipSuccess) return e;
  const size_t nx = 2 * (size_t)d.d_model, np = m->proj_rows, no = m->V + 8 * (size_t)d.n_heads;
  e = hipMalloc(&m->xchg, exchange_words(m) * sizeof(uint64_t));
  if (e != hipSuccess) return e;
  e = hipMemset(m->xchg, 0, exchange_words(m) * sizeof(uint64_t));
  if (e != hipSuccess) return e;
  e = hipMalloc(&m->err, 256);
  if (e != hipSuccess) return e;
  e = hipMemset(m->err, 0, 256);
  if (e != hipSuccess) return e;
  e = hipHostMalloc((void**)&m->err_host, 256, hipHostMallocDefault);
  if (e != hipSuccess) return e;
  *(volatile int*)m->err_host = 0;
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  PersistParams& p = m->pp;
  p.n_layers = d.n_layers; p.D = d.d_model; p.H = d.n_heads; p.dk = d.d_k; p.dv = d.d_v;
  p.C = m->C; p.rank = d.rank_f; p.proj_rows = m->proj_rows;
  p.gate_safe = safe ? 1 : 0;
  p.gate_lb = d.gate_lb;
  const int rows[6] = {m->Kq, m->Kq, m->V, d.rank_f, d.rank_g, d.n_heads};
  int first = 0;
  for (int i = 0; i < 6; ++i) { p.seg_first[i] = first; first += rows[i]; }
  p.eps = d.norm_eps; p.l2_eps = d.l2_eps; p.q_scale = m->q_scale;
  p.layers = m->d_layers;
  p.xbuf = m->xchg; p.pbuf = p.xbuf + nx; p.obuf = p.pbuf + np; p.flags = p.obuf + no;
  p.err = m->err;
  p.err_host = m->err_host;
  int dev = 0, khz = 0;
  e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return e;
  m->wall_khz = khz > 0 ? khz : 100000;
  set_wait_limit(m, 0);
  p.o_first_block = ob0; p.o_blocks = nob;
  p.q_blocks = m->C / 48;
  m->pers_blocks = nb;
  m->pers_ok = true;
  // the per-layer path reads the same copies (and never the caller's buffers again); an
  // MXFP4, scalar- or lower-bounded-gate stack keeps its per-layer kernels on the caller's
  // buffers (their matrix-core gates compute KDA's form)
  for (int l = 0; l < d.n_layers && !mx4 && !scal && !safe; ++l) {
    m->layers[l].pw = host[l].pw;
    m->layers[l].pd = host[l].pd;
    m->layers[l].ow = host[l].ow;
    m->layers[l].od = host[l].od;
    m->layers[l].fbw = host[l].fbw;
    m->layers[l].fbd = host[l].fbd;
    m->layers[l].gbw = host[l].gbw;
    m->layers[l].gbd = host[l].gbd;
  }
  return hipSuccess;
}

int reset_exchange(kda_model* m) {
  KDA_HIP(hipDeviceSynchronize());
  KDA_HIP(hipMemset(m->xchg, 0, exchange_words(m) * sizeof(uint64_t)));
  KDA_HIP(hipMemset(m->err, 0, 256));
  KDA_HIP(hipDeviceSynchronize());
  *(volatile int*)m->err_host = 0;
  m->epoch = 0;
  return KDA_OK;
}

// ---- a device workspace for callers that cannot allocate (kda_decode_step_static) ----
// One array per GPU for the life of the process, shared by every model and call on that
// GPU.  In host code `scratch` names a host-side stand-in, not device memory: its device
// address comes from hipGetSymbolAddress, taken once per device (with that device
// current) and kept in g_scratch_ptr; only that address is ever passed to a kernel.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
constexpr int kMaxScratchDevices = 64;
static __device__ __attribute__((used)) __align__(256) char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's scratch address (looked up on its first use on that device).
int static_scratch(void** out) {
  int dev = 0;
  KDA_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(KDA_E_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KDA_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

// Sequential-scan prefill: tokens in blocks of Tc per sequence (B * Tc <= 64 columns, the
// matrix-core projections' range, or Tc = 1 for wide batches); per block the per-layer
// workspace of B * Tc columns, the activated q|k|v, and staging rows for the block's input
// and output ([B][Tc][D] each).
struct ScanLayout {
  int Tc = 1;
  WsLayout wl;
  size_t act = 0, xs = 0, ys = 0, total = 0;
};

ScanLayout scan_layout(const kda_model* m, int64_t B, int64_t L) {
  ScanLayout s;
  s.Tc = (int)std::max<int64_t>(1, std::min<int64_t>(L, 64 / B));
  const int64_t N = B * s.Tc;
  s.wl = ws_layout(m, N);
  size_t off = s.wl.total;
  s.act = off; off = align_up(off + (size_t)N * m->C * 4, 256);
  s.xs = off;  off = align_up(off + (size_t)N * m->d.d_model * 4, 256);
  s.ys = off;  off = align_up(off + (size_t)N * m->d.d_model * 4, 256);
  s.total = off;
  return s;
}

// A one-launch step whose wait between blocks ran out left the caller's state partly
// advanced; until kda_model_status has reported it, every call that reads or writes a state
// on this model is refused (the kernel itself also leaves at once while the device word is
// set, for steps enqueued before the host saw it).
int check_poison(const kda_model* m) {
  if (m->err_host && *(volatile const int*)m->err_host)
    return fail(KDA_E_HIP, "an earlier one-launch decode step on this model timed out in a wait "
                "between blocks; its state is invalid: call kda_model_status to reset the model");
  return KDA_OK;
}

// ---- host-side packing (kda_pack from host memory), the same rules as the device kernels
void host_pack_bf16(const float* src, uint16_t* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t b;
    std::memcpy(&b, src + i, 4);
    if ((b & 0x7fffffffu) > 0x7f800000u) dst[i] = (uint16_t)((b >> 16) | 0x40u);
    else dst[i] = (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
  }
}

// Q8_0 per block of 32: amax, d = fp32(amax / 127), d16 = fp16 round-to-nearest-even of d,
// q = clamp(round-half-away(fp32(x / d16)), -127, 127), all q = 0 when d16 == 0; stored as
// q + 128 with the scale plane at q8_scale_offset.
void host_pack_q8_0(const float* src, int64_t rows, int64_t cols, uint8_t* dst) {
  const int64_t nb = cols / 32;
  uint16_t* dplane = reinterpret_cast<uint16_t*>(dst + q8_scale_offset(rows, cols));
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < nb; ++j) {
      const float* x = src + r * cols + j * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) amax = std::fmax(amax, std::fabs(x[i]));
      const volatile float d = amax / 127.0f;
      const _Float16 h = (_Float16)d;
      const float dq = (float)h;
      uint8_t* q = dst + r * cols + j * 32;
      for (int i = 0; i < 32; ++i) {
        float t = 0.0f;
        if (dq != 0.0f) {
          const volatile float ratio = x[i] / dq;
          t = std::fmin(std::fmax(std::round(ratio), -127.0f), 127.0f);
        }
        q[i] = (uint8_t)((int)t + 128);
      }
      uint16_t bits;
      std::memcpy(&bits, &h, 2);
      dplane[r * nb + j] = bits;
    }
}

// MXFP4 on the host, the same rule as the device kernel pack_mxfp4 (pack.hip).
uint32_t host_e2m1_code(float v) {
  const float a = std::fabs(v);
  const uint32_t idx = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                       (a >= 3.5f) + (a > 5.0f);
  return ((v < 0.0f && idx > 0) ? 8u : 0u) | idx;
}

void host_pack_mxfp4(const float* src, int64_t rows, int64_t cols, uint8_t* dst) {
  const int64_t nb = cols / 32;
  uint8_t* eplane = dst + mx4_scale_offset(rows, cols);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < nb; ++j) {
      const float* x = src + r * cols + j * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) amax = std::fmax(amax, std::fabs(x[i]));
      int s = -127;
      if (amax > 0.0f) {
        int ex = 0;
        (void)std::frexp(amax, &ex);
        s = std::min(std::max(ex - 1 - 2, -127), 127);
      }
      uint8_t* q = dst + r * (cols / 2) + j * 16;
      for (int i = 0; i < 16; ++i)
        q[i] = (uint8_t)(host_e2m1_code(std::ldexp(x[2 * i], -s)) |
                         (host_e2m1_code(std::ldexp(x[2 * i + 1], -s)) << 4));
      eplane[r * nb + j] = (uint8_t)(s + 127);
    }
}

}  // namespace

// =======================================================================================
extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_E_ARG: return "invalid argument";
    case KDA_E_SHAPE: return "unsupported or inconsistent shape";
    case KDA_E_ALIGN: return "device pointer not 16-byte aligned";
    case KDA_E_DTYPE: return "unsupported data type";
    case KDA_E_WORKSPACE: return "workspace too small";
    case KDA_E_HIP: return "HIP runtime error";
    case KDA_E_UNSUPPORTED: return "unsupported";
    default: return "unknown status";
  }
}

const char* kda_last_error(void) { return g_err.c_str(); }

size_t kda_packed_bytes(int dtype, int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  switch (dtype) {
    case KDA_F32: return (size_t)rows * cols * 4;
    case KDA_BF16: return (size_t)rows * cols * 2;
    case KDA_Q8_0:
      if (cols % 32) return 0;
      return q8_scale_offset(rows, cols) + (size_t)rows * (cols / 32) * 2;
    case KDA_MXFP4:
      if (cols % 32) return 0;
      return mx4_scale_offset(rows, cols) + (size_t)rows * (cols / 32);
    default: return 0;
  }
}

int kda_pack(int dtype, const float* src_host, int64_t rows, int64_t cols, void* dst_dev,
             void* stream) {
  if (dtype < KDA_F32 || dtype > KDA_MXFP4) return fail(KDA_E_DTYPE, "unknown dtype %d", dtype);
  if (!src_host || !dst_dev) return fail(KDA_E_ARG, "null pointer");
  if (rows <= 0 || cols <= 0) return fail(KDA_E_SHAPE, "rows/cols must be positive");
  if ((dtype == KDA_Q8_0 || dtype == KDA_MXFP4) && cols % 32)
    return fail(KDA_E_SHAPE, "block formats need cols %% 32 == 0");
  if (!aligned16(dst_dev)) return fail(KDA_E_ALIGN, "dst_dev must be 16-byte aligned");
  const size_t bytes = kda_packed_bytes(dtype, rows, cols);
  std::vector<uint8_t> buf(bytes, 0);
  if (dtype == KDA_F32) std::memcpy(buf.data(), src_host, (size_t)rows * cols * 4);
  else if (dtype == KDA_BF16) host_pack_bf16(src_host, reinterpret_cast<uint16_t*>(buf.data()), rows * cols);
  else if (dtype == KDA_MXFP4) host_pack_mxfp4(src_host, rows, cols, buf.data());
  else host_pack_q8_0(src_host, rows, cols, buf.data());
  hipStream_t s = (hipStream_t)stream;
  KDA_HIP(hipMemcpyAsync(dst_dev, buf.data(), bytes, hipMemcpyHostToDevice, s));
  KDA_HIP(hipStreamSynchronize(s));
  return KDA_OK;
}

int kda_pack_device(int dtype, const float* src_dev, int64_t rows, int64_t cols, void* dst_dev,
                    void* stream) {
  if (dtype < KDA_F32 || dtype > KDA_MXFP4) return fail(KDA_E_DTYPE, "unknown dtype %d", dtype);
  if (!src_dev || !dst_dev) return fail(KDA_E_ARG, "null pointer");
  if (rows <= 0 || cols <= 0) return fail(KDA_E_SHAPE, "rows/cols must be positive");
  if ((dtype == KDA_Q8_0 || dtype == KDA_MXFP4) && cols % 32)
    return fail(KDA_E_SHAPE, "block formats need cols %% 32 == 0");
  if (!aligned16(src_dev) || !aligned16(dst_dev)) return fail(KDA_E_ALIGN, "pointers must be 16-byte aligned");
  KDA_HIP(launch_pack(dtype, src_dev, rows, cols, dst_dev, (hipStream_t)stream));
  return KDA_OK;
}

int kda_unpack_q8_0(const void* packed_dev, int64_t rows, int64_t cols, uint16_t* d16_host,
                    int8_t* qs_host, void* stream) {
  if (!packed_dev || !d16_host || !qs_host) return fail(KDA_E_ARG, "null pointer");
  if (rows <= 0 || cols <= 0 || cols % 32) return fail(KDA_E_SHAPE, "bad Q8_0 shape");
  const size_t bytes = kda_packed_bytes(KDA_Q8_0, rows, cols);
  std::vector<uint8_t> buf(bytes);
  hipStream_t s = (hipStream_t)stream;
  KDA_HIP(hipMemcpyAsync(buf.data(), packed_dev, bytes, hipMemcpyDeviceToHost, s));
  KDA_HIP(hipStreamSynchronize(s));
  const size_t n = (size_t)rows * cols;
  for (size_t i = 0; i < n; ++i) qs_host[i] = (int8_t)((int)buf[i] - 128);
  std::memcpy(d16_host, buf.data() + q8_scale_offset(rows, cols), n / 32 * 2);
  return KDA_OK;
}

int kda_unpack_mxfp4(const void* packed_dev, int64_t rows, int64_t cols, uint8_t* e8m0_host,
                     uint8_t* codes_host, void* stream) {
  if (!packed_dev || !e8m0_host || !codes_host) return fail(KDA_E_ARG, "null pointer");
  if (rows <= 0 || cols <= 0 || cols % 32) return fail(KDA_E_SHAPE, "bad MXFP4 shape");
  const size_t bytes = kda_packed_bytes(KDA_MXFP4, rows, cols);
  std::vector<uint8_t> buf(bytes);
  hipStream_t s = (hipStream_t)stream;
  KDA_HIP(hipMemcpyAsync(buf.data(), packed_dev, bytes, hipMemcpyDeviceToHost, s));
  KDA_HIP(hipStreamSynchronize(s));
  const size_t n = (size_t)rows * cols;
  for (size_t i = 0; i < n; ++i) codes_host[i] = (buf[i / 2] >> (4 * (i & 1))) & 0x0Fu;
  std::memcpy(e8m0_host, buf.data() + mx4_scale_offset(rows, cols), n / 32);
  return KDA_OK;
}

int kda_unpack_q8_0_device(const void* packed_dev, int64_t rows, int64_t cols, uint16_t* d16_dev,
                           int8_t* qs_dev, void* stream) {
  if (!packed_dev || !d16_dev || !qs_dev) return fail(KDA_E_ARG, "null pointer");
  if (rows <= 0 || cols <= 0 || cols % 32) return fail(KDA_E_SHAPE, "bad Q8_0 shape");
  KDA_HIP(launch_unpack_q8(packed_dev, rows, cols, d16_dev, qs_dev, (hipStream_t)stream));
  return KDA_OK;
}

int kda_model_create(const kda_dims* dims, const kda_layer* layers, kda_model** out) {
  if (!dims || !layers || !out) return fail(KDA_E_ARG, "null pointer");
  *out = nullptr;
  const kda_dims& d = *dims;
  if (d.wtype < KDA_F32 || d.wtype > KDA_MXFP4) return fail(KDA_E_DTYPE, "unknown wtype %d", d.wtype);
  if (d.n_layers < 1 || d.n_heads < 1 || d.d_model < 1) return fail(KDA_E_SHAPE, "sizes must be positive");
  if (d.d_k != d.d_v) return fail(KDA_E_SHAPE, "d_k must equal d_v");
  if (d.d_k != 64 && d.d_k != 128) return fail(KDA_E_SHAPE, "d_k must be 64 or 128");
  if (d.conv_k != 4) return fail(KDA_E_SHAPE, "conv_k must be 4");
  if (d.rank_f < 1 || d.rank_g < 1 || d.rank_f > 256 || d.rank_g > 256)
    return fail(KDA_E_SHAPE, "ranks must be in 1..256");
  const int gran = (d.wtype == KDA_Q8_0 || d.wtype == KDA_MXFP4) ? 32 : (d.wtype == KDA_BF16 ? 8 : 4);
  if (d.d_model % gran || d.rank_f % gran || d.rank_g % gran || (d.n_heads * d.d_v) % gran)
    return fail(KDA_E_SHAPE, "input dims must be multiples of %d for this weight type", gran);
  if (d.d_model % 4) return fail(KDA_E_SHAPE, "d_model %% 4 != 0");
  if (d.d_model > kGemvKMax || d.n_heads * d.d_v > kGemvKMax)
    return fail(KDA_E_SHAPE, "d_model and n_heads*d_v must be <= %d", kGemvKMax);
  if (d.n_heads > kGemvMaxHeads) return fail(KDA_E_SHAPE, "n_heads must be <= %d", kGemvMaxHeads);
  if (!head_supported(d.d_k, d.wtype, d.rank_f, d.rank_g))
    return fail(KDA_E_SHAPE, "low ranks %d/%d unsupported for this weight type (need rank_f == rank_g, "
                "a power-of-two count of 16-byte chunks per row)", d.rank_f, d.rank_g);
  if (!(d.norm_eps >= 0.f) || !(d.l2_eps >= 0.f)) return fail(KDA_E_ARG, "eps must be >= 0");
  if (d.gate < KDA_GATE_KDA || d.gate > KDA_GATE_SCALAR) return fail(KDA_E_ARG, "unknown gate form %d", d.gate);
  if (d.gate == KDA_GATE_SAFE && !(d.gate_lb < 0.f && d.gate_lb > -1e30f))
    return fail(KDA_E_ARG, "the safe gate needs a finite gate_lb < 0");
  kda_model* m = new kda_model();
  m->d = d;
  m->Kq = d.n_heads * d.d_k;
  m->V = d.n_heads * d.d_v;
  m->C = 2 * m->Kq + m->V;
  m->proj_rows = m->C + d.rank_f + d.rank_g + d.n_heads;
  m->proj_stride = (int)align_up(m->proj_rows, 4);
  m->q_scale = (float)(1.0 / std::sqrt((double)d.d_k));
  const int64_t D = d.d_model;
  for (int l = 0; l < d.n_layers; ++l) {
    const kda_layer& s = layers[l];
    const void* ptrs[] = {s.wq, s.wk, s.wv, s.wo, s.fa, s.fb, s.wbeta, s.ga, s.gb,
                          s.conv_w, s.a_log, s.dt_bias};
    for (const void* p : ptrs) {
      if (!p) { delete m; return fail(KDA_E_ARG, "layer %d: null parameter pointer", l); }
      if (!aligned16(p)) { delete m; return fail(KDA_E_ALIGN, "layer %d: parameter not 16-byte aligned", l); }
    }
    LayerDev L;
    L.wq = packed_view(s.wq, d.wtype, m->Kq, D);
    L.wk = packed_view(s.wk, d.wtype, m->Kq, D);
    L.wv = packed_view(s.wv, d.wtype, m->V, D);
    L.wo = packed_view(s.wo, d.wtype, D, m->V);
    L.fa = packed_view(s.fa, d.wtype, d.rank_f, D);
    L.fb = packed_view(s.fb, d.wtype, d.gate == KDA_GATE_SCALAR ? d.n_heads : m->Kq, d.rank_f);
    L.wbeta = packed_view(s.wbeta, d.wtype, d.n_heads, D);
    L.ga = packed_view(s.ga, d.wtype, d.rank_g, D);
    L.gb = packed_view(s.gb, d.wtype, m->V, d.rank_g);
    L.conv_w = s.conv_w;
    L.a_log = s.a_log;
    L.dt_bias = s.dt_bias;
    L.o_norm_w = s.o_norm_w;
    m->layers.push_back(L);
  }
  {
    // the static scratch's address on this device, taken once here (the library's set-up
    // call) so that kda_decode_step_static finds it ready
    void* sp = nullptr;
    const int r = static_scratch(&sp);
    if (r) { delete m; return r; }
  }
  hipError_t e = hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking);
  if (e == hipSuccess) e = persist_setup(m, layers);
  if (e != hipSuccess) {
    kda_model_destroy(m);
    return fail(KDA_E_HIP, "model setup: %s", hipGetErrorString(e));
  }
  *out = m;
  return KDA_OK;
}

void kda_model_destroy(kda_model* m) {
  if (!m) return;
  drop_graph(m);
  if (m->d_layers) (void)hipFree(m->d_layers);
  if (m->mma_w) (void)hipFree(m->mma_w);
  if (m->dtb_rep) (void)hipFree(m->dtb_rep);
  if (m->xchg) (void)hipFree(m->xchg);
  if (m->err) (void)hipFree(m->err);
  if (m->err_host) (void)hipHostFree(m->err_host);
  for (auto& t : m->pool) {
    (void)hipEventDestroy(t.a);
    (void)hipEventDestroy(t.b);
  }
  if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
  delete m;
}

int kda_model_set_option(kda_model* m, int option, int64_t value) {
  if (!m) return fail(KDA_E_ARG, "null model");
  switch (option) {
    case KDA_OPT_GRAPH:
      m->use_graph = value != 0;
      if (!m->use_graph) drop_graph(m);
      return KDA_OK;
    case KDA_OPT_TIMING:
      m->timing = value != 0;
      return KDA_OK;
    case KDA_OPT_PERSISTENT:
      m->use_persist = value != 0;
      return KDA_OK;
    case KDA_OPT_WAIT_US:
      if (m->pers_ok) set_wait_limit(m, value);
      return KDA_OK;
    case KDA_OPT_COOPERATIVE:
      m->coop = value != 0;
      return KDA_OK;
    default:
      return fail(KDA_E_ARG, "unknown option %d", option);
  }
}

int kda_model_status(kda_model* m) {
  if (!m) return fail(KDA_E_ARG, "null model");
  KDA_HIP(hipDeviceSynchronize());
  if (!m->pers_ok) return KDA_OK;
  int err = 0;
  KDA_HIP(hipMemcpy(&err, m->err, sizeof(int), hipMemcpyDeviceToHost));
  if (err || *(volatile int*)m->err_host) {
    int r = reset_exchange(m);
    if (r) return r;
    return fail(KDA_E_HIP, "one-launch decode: a wait between blocks timed out; outputs of "
                "the affected steps are invalid");
  }
  return KDA_OK;
}

int kda_model_query(const kda_model* m, int what) {
  if (!m) return -1;
  switch (what) {
    case KDA_Q_PERSISTENT: return m->pers_ok ? m->pers_blocks : 0;
    case KDA_Q_OWNS_WEIGHTS:
      return m->mma_w && m->d.wtype == KDA_Q8_0 && m->d.gate == KDA_GATE_KDA ? 1 : 0;
    default: return -1;
  }
}

int kda_timing_query(kda_model* m, int kind, double* total_ms, int64_t* launches, int reset) {
  if (!m || kind < 0 || kind >= KDA_K_COUNT) return fail(KDA_E_ARG, "bad timing query");
  int r = flush_timing(m);
  if (r) return r;
  if (total_ms) *total_ms = m->total_ms[kind];
  if (launches) *launches = m->count[kind];
  if (reset) {
    for (int i = 0; i < KDA_K_COUNT; ++i) { m->total_ms[i] = 0; m->count[i] = 0; }
  }
  return KDA_OK;
}

size_t kda_workspace_bytes(const kda_model* m, int op, int32_t batch, int64_t tokens) {
  if (!m || batch < 1 || tokens < 1) return 0;
  if (op == KDA_OP_DECODE) return ws_layout(m, batch).total;
  if (op == KDA_OP_VERIFY) return ws_layout(m, (int64_t)batch * tokens).total;
  if (op == KDA_OP_PREFILL) return pf_layout(m, batch, tokens).total;
  if (op == KDA_OP_SCAN) return scan_layout(m, batch, tokens).total;
  return 0;
}

}  // extern "C"

namespace {

// One decode token for every sequence; `active` (device [B] or null) masks sequences whose
// state and window stay as they are.  A masked step never takes the one-launch kernel.
int decode_impl(kda_model* m, const float* x_dev, float* y_dev, const kda_state* st,
                const int32_t* active, void* ws_dev, size_t ws_bytes, void* stream,
                bool eager = false) {
  if (!m || !x_dev || !y_dev || !ws_dev) return fail(KDA_E_ARG, "null pointer");
  int r = check_state(m, st);
  if (r) return r;
  if (!aligned16(x_dev) || !aligned16(y_dev) || !aligned16(ws_dev)) return fail(KDA_E_ALIGN, "unaligned pointer");
  if (active && ((uintptr_t)active & 3u)) return fail(KDA_E_ALIGN, "active mask not 4-byte aligned");
  if (ws_bytes < ws_layout(m, st->batch).total)
    return fail(KDA_E_WORKSPACE, "workspace %zu < %zu", ws_bytes, ws_layout(m, st->batch).total);
  r = check_poison(m);
  if (r) return r;
  hipStream_t s = (hipStream_t)stream;
  char* ws = static_cast<char*>(ws_dev);
  r = flush_state(m, st, s, true, nullptr, eager);
  if (r) return r;
  if (!active && m->use_persist && m->pers_ok && st->batch == 1) {
    if (m->epoch >= 0x7fffffffu / (uint32_t)m->d.n_layers) {
      r = reset_exchange(m);
      if (r) return r;
    }
    PersistParams p = m->pp;
    p.S = st->S_dev; p.win = st->conv_dev; p.x_in = x_dev; p.y_out = y_dev;
    p.epoch = ++m->epoch;
    return timed(m, KDA_K_STEP, s, m->timing && !eager,
                 [&] { return launch_persistent(p, m->pers_blocks, m->coop, s); });
  }
  // (eager: no graph capture or instantiation and no timing events, which allocate)
  if (eager) return enqueue_decode(m, x_dev, y_dev, st, ws, s, false, active);
  if (!m->use_graph || m->timing) return enqueue_decode(m, x_dev, y_dev, st, ws, s, m->timing, active);

  const std::vector<uintptr_t> key = {(uintptr_t)x_dev, (uintptr_t)y_dev, (uintptr_t)st->S_dev,
                                      (uintptr_t)st->conv_dev, (uintptr_t)ws_dev,
                                      (uintptr_t)active, (uintptr_t)st->batch};
  return run_graph(m, kGraphDecode, key, s, [&](hipStream_t cs) {
    return enqueue_decode(m, x_dev, y_dev, st, ws, cs, false, active);
  });
}

}  // namespace

extern "C" {

int kda_decode_step(kda_model* m, const float* x_dev, float* y_dev, const kda_state* st,
                    void* ws_dev, size_t ws_bytes, void* stream) {
  return decode_impl(m, x_dev, y_dev, st, nullptr, ws_dev, ws_bytes, stream);
}

int kda_decode_step_static(kda_model* m, const float* x_dev, float* y_dev, const kda_state* st,
                           void* stream) {
  if (!m) return fail(KDA_E_ARG, "null model");
  int r = check_state(m, st);
  if (r) return r;
  const size_t need = ws_layout(m, st->batch).total;
  if (need > kStaticScratchBytes)
    return fail(KDA_E_WORKSPACE, "batch %d needs %zu workspace bytes, more than the %zu of the "
                "static scratch; use kda_decode_step with a workspace", st->batch, need,
                kStaticScratchBytes);
  void* ws = nullptr;
  r = static_scratch(&ws);
  if (r) return r;
  return decode_impl(m, x_dev, y_dev, st, nullptr, ws, kStaticScratchBytes, stream, true);
}

int kda_decode_step_masked(kda_model* m, const float* x_dev, float* y_dev, const kda_state* st,
                           const int32_t* active_dev, void* ws_dev, size_t ws_bytes,
                           void* stream) {
  if (!active_dev) return fail(KDA_E_ARG, "null active mask");
  return decode_impl(m, x_dev, y_dev, st, active_dev, ws_dev, ws_bytes, stream);
}

size_t kda_verify_log_bytes(const kda_model* m, int32_t batch, int32_t T) {
  if (!m || batch < 1 || T < 1) return 0;
  return log_hdr_bytes(batch) + 2 * log_half_bytes(m, batch, T);
}

int kda_verify_steps(kda_model* m, const float* x_dev, int32_t T, float* y_dev,
                     const kda_state* st, void* log_dev, size_t log_bytes, void* ws_dev,
                     size_t ws_bytes, void* stream) {
  if (!m || !x_dev || !y_dev || !log_dev || !ws_dev) return fail(KDA_E_ARG, "null pointer");
  int r = check_state(m, st);
  if (r) return r;
  if (T < 1 || T > 8) return fail(KDA_E_SHAPE, "T must be in 1..8");
  if (!aligned16(x_dev) || !aligned16(y_dev) || !aligned16(log_dev) || !aligned16(ws_dev))
    return fail(KDA_E_ALIGN, "unaligned pointer");
  const int B = st->batch;
  if (log_half_cap(log_bytes, B) < log_half_bytes(m, B, T))
    return fail(KDA_E_WORKSPACE, "log of %zu bytes is smaller than a verify of B=%d, T=%d needs (%zu)",
                log_bytes, B, T, kda_verify_log_bytes(m, B, T));
  WsLayout wl = ws_layout(m, (int64_t)B * T);
  if (ws_bytes < wl.total) return fail(KDA_E_WORKSPACE, "workspace %zu < %zu", ws_bytes, wl.total);
  r = check_poison(m);
  if (r) return r;
  hipStream_t s = (hipStream_t)stream;
  char* ws = static_cast<char*>(ws_dev);
  // commits pending on this state through other logs are applied first; one recorded on
  // this log is folded into this verify
  const LogRec* mine = find_log(m, st, log_dev, log_bytes);
  r = flush_state(m, st, s, true, mine);
  if (r) return r;
  r = flush_log(m, log_dev, st, s);
  if (r) return r;
  LogRec* rc = add_log(m, st, log_dev, log_bytes);
  if (!rc) return fail(KDA_E_ARG, "%zu commits are pending on this model: apply some with kda_state_flush",
                       kMaxLogs);
  const bool fold = rc->pend_half >= 0;
  const int half = fold ? 1 - rc->pend_half : 0;
  const int pT = rc->pend_T, phalf = rc->pend_half;
  auto enqueue = [&](hipStream_t cs, bool rec) {
    for (int l = 0; l < m->d.n_layers; ++l) {
      const float* xin = (l == 0 || !m->d.prenorm_residual) ? x_dev : y_dev;
      const LogLayer ll = log_layer(m, log_dev, log_bytes, B, T, half, l);
      FoldSrc fs;
      if (fold) {
        const LogLayer pl = log_layer(m, log_dev, log_bytes, B, pT, phalf, l);
        fs.proj = pl.proj;
        fs.ag = pl.ag;
        fs.act = pl.act;
        fs.ntok = static_cast<const int*>(log_dev);
        fs.T = pT;
      }
      const int rr = enqueue_layer(m, l, xin, y_dev, B, T, st->S_dev + l * state_layer_stride(m, B),
                                   st->conv_dev + l * win_layer_stride(m, B), ll.proj, ll.ag,
                                   ll.act, wl, ws, false, cs, rec, nullptr, false,
                                   fold ? &fs : nullptr);
      if (rr) return rr;
    }
    return (int)KDA_OK;
  };
  if (!m->use_graph || m->timing) {
    r = enqueue(s, m->timing);
  } else {
    const std::vector<uintptr_t> key = {(uintptr_t)x_dev, (uintptr_t)y_dev, (uintptr_t)st->S_dev,
                                        (uintptr_t)st->conv_dev, (uintptr_t)log_dev,
                                        (uintptr_t)log_bytes, (uintptr_t)ws_dev, (uintptr_t)B,
                                        (uintptr_t)T, (uintptr_t)fold, (uintptr_t)pT};
    r = run_graph(m, half ? kGraphVerifyOdd : kGraphVerify, key, s,
                  [&](hipStream_t cs) { return enqueue(cs, false); });
  }
  rc = find_log(m, st, log_dev, log_bytes);
  rc->pend_half = -1;
  rc->last_half = r ? -1 : half;
  rc->last_T = T;
  return r;
}

int kda_verify_commit(kda_model* m, const kda_state* st, const void* log_dev, size_t log_bytes,
                      int32_t T, const int32_t* accept_dev, void* stream) {
  if (!m || !log_dev || !accept_dev) return fail(KDA_E_ARG, "null pointer");
  int r = check_state(m, st);
  if (r) return r;
  if (T < 1 || T > 8) return fail(KDA_E_SHAPE, "T must be in 1..8");
  const int B = st->batch;
  if (log_half_cap(log_bytes, B) < log_half_bytes(m, B, T))
    return fail(KDA_E_WORKSPACE, "log of %zu bytes is smaller than a verify of B=%d, T=%d writes (%zu)",
                log_bytes, B, T, kda_verify_log_bytes(m, B, T));
  if (!aligned16(log_dev) || ((uintptr_t)accept_dev & 3u)) return fail(KDA_E_ALIGN, "unaligned pointer");
  r = check_poison(m);
  if (r) return r;
  LogRec* rc = find_log(m, st, log_dev, log_bytes);
  if (!rc || rc->last_half < 0 || rc->last_T != T)
    return fail(KDA_E_ARG, "no verify of T=%d tokens on this state and log to commit (a commit "
                "follows its verify, with no other call on the state in between)", T);
  // the accepted lengths go to the log header: the caller's buffer is free again once the
  // stream has passed this point
  KDA_HIP(hipMemcpyAsync(const_cast<void*>(log_dev), accept_dev, (size_t)B * 4,
                         hipMemcpyDeviceToDevice, (hipStream_t)stream));
  rc->pend_half = rc->last_half;
  rc->pend_T = T;
  rc->last_half = -1;
  return KDA_OK;
}

int kda_state_flush(kda_model* m, const kda_state* st, void* stream) {
  if (!m) return fail(KDA_E_ARG, "null model");
  int r = check_state(m, st);
  if (r) return r;
  r = check_poison(m);
  if (r) return r;
  return flush_state(m, st, (hipStream_t)stream, false);
}

int kda_prefill_scan(kda_model* m, const float* x_dev, int64_t L, float* y_dev,
                     const kda_state* st, void* ws_dev, size_t ws_bytes, void* stream) {
  if (!m || !x_dev || !y_dev || !ws_dev) return fail(KDA_E_ARG, "null pointer");
  int r = check_state(m, st);
  if (r) return r;
  if (L < 1 || L > (1 << 30)) return fail(KDA_E_SHAPE, "L must be >= 1");
  if (!aligned16(x_dev) || !aligned16(y_dev) || !aligned16(ws_dev)) return fail(KDA_E_ALIGN, "unaligned pointer");
  const int B = st->batch;
  const ScanLayout sl = scan_layout(m, B, L);
  if (ws_bytes < sl.total) return fail(KDA_E_WORKSPACE, "workspace %zu < %zu", ws_bytes, sl.total);
  r = check_poison(m);
  if (r) return r;
  hipStream_t s = (hipStream_t)stream;
  r = flush_state(m, st, s, true);
  if (r) return r;
  char* ws = static_cast<char*>(ws_dev);
  const int D = m->d.d_model;
  float* xs = reinterpret_cast<float*>(ws + sl.xs);
  float* ys = reinterpret_cast<float*>(ws + sl.ys);
  float* proj = reinterpret_cast<float*>(ws + sl.wl.proj);
  float* ag = reinterpret_cast<float*>(ws + sl.wl.ag);
  float* act = reinterpret_cast<float*>(ws + sl.act);
  for (int64_t t0 = 0; t0 < L; t0 += sl.Tc) {
    const int T = (int)std::min<int64_t>(sl.Tc, L - t0);
    // the block's rows [B][T][D], gathered from x [B][L][D]
    KDA_HIP(hipMemcpy2DAsync(xs, (size_t)T * D * 4, x_dev + t0 * D, (size_t)L * D * 4,
                             (size_t)T * D * 4, B, hipMemcpyDeviceToDevice, s));
    for (int l = 0; l < m->d.n_layers; ++l) {
      const float* xin = (l == 0 || !m->d.prenorm_residual) ? xs : ys;
      r = enqueue_layer(m, l, xin, ys, B, T, st->S_dev + l * state_layer_stride(m, B),
                        st->conv_dev + l * win_layer_stride(m, B), proj, ag, act, sl.wl, ws,
                        true, s, m->timing, nullptr, true);
      if (r) return r;
    }
    KDA_HIP(hipMemcpy2DAsync(y_dev + t0 * D, (size_t)L * D * 4, ys, (size_t)T * D * 4,
                             (size_t)T * D * 4, B, hipMemcpyDeviceToDevice, s));
  }
  return KDA_OK;
}

int kda_conv_window_canonical(kda_model* m, const kda_state* st, float* out_dev, void* stream) {
  if (!m || !out_dev) return fail(KDA_E_ARG, "null pointer");
  int r = check_state(m, st);
  if (r) return r;
  if (!aligned16(out_dev)) return fail(KDA_E_ALIGN, "unaligned pointer");
  r = check_poison(m);
  if (r) return r;
  r = flush_state(m, st, (hipStream_t)stream, false);
  if (r) return r;
  // the device window is already [n_layers][B][conv_k - 1][C], oldest token first
  const size_t n = (size_t)m->d.n_layers * win_layer_stride(m, st->batch);
  KDA_HIP(hipMemcpyAsync(out_dev, st->conv_dev, n * sizeof(float), hipMemcpyDeviceToDevice,
                         (hipStream_t)stream));
  return KDA_OK;
}

int kda_prefill_chunked(kda_model* m, const void* x_dev, int x_dtype, int64_t L,
                        int32_t chunk, float* y_dev, const kda_state* st, void* ws_dev,
                        size_t ws_bytes, void* stream) {
  if (!m || !x_dev || !y_dev || !ws_dev) return fail(KDA_E_ARG, "null pointer");
  int r = check_state(m, st);
  if (r) return r;
  const kda_dims& d = m->d;
  if (d.n_layers != 1 || d.prenorm_residual)
    return fail(KDA_E_UNSUPPORTED, "chunked prefill takes a single layer without pre-norm residual");
  if (d.wtype != KDA_BF16) return fail(KDA_E_DTYPE, "chunked prefill needs BF16 weights (MFMA operands)");
  if (x_dtype != KDA_BF16 && x_dtype != KDA_F32) return fail(KDA_E_DTYPE, "x must be BF16 or F32");
  if (chunk != kChunk) return fail(KDA_E_SHAPE, "chunk must be %d", kChunk);
  if (L < 1 || L > (1 << 30)) return fail(KDA_E_SHAPE, "L must be >= 1");
  if (d.d_model % 64 || d.rank_g % 64 || m->V % 64)
    return fail(KDA_E_SHAPE, "prefill GEMMs need d_model, rank_g and H*d_v multiples of 64");
  if (d.rank_f != 64 && d.rank_f != 128) return fail(KDA_E_SHAPE, "chunked prefill needs rank_f 64 or 128");
  if (!aligned16(x_dev) || !aligned16(y_dev) || !aligned16(ws_dev)) return fail(KDA_E_ALIGN, "unaligned pointer");
  const int B = st->batch;
  const PfLayout wl = pf_layout(m, B, L);
  if (ws_bytes < wl.total) return fail(KDA_E_WORKSPACE, "workspace %zu < %zu", ws_bytes, wl.total);
  r = check_poison(m);
  if (r) return r;
  hipStream_t s = (hipStream_t)stream;
  r = flush_state(m, st, s, true);
  if (r) return r;
  char* ws = static_cast<char*>(ws_dev);
  const LayerDev& Ly = m->layers[0];
  const int64_t M = (int64_t)B * L;
  const bool rec = m->timing;
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };

  // P1: fused input projections [q|k|v|f_a|g_a|beta] on matrix cores
  GemmParams g;
  auto U16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
  if (x_dtype == KDA_F32) {
    uint16_t* xh = U16(wl.xs);
    uint16_t* xl = xh + (size_t)M * d.d_model;
    r = timed(m, KDA_K_GEMM, s, rec, [&] {
      return launch_split_planes(static_cast<const float*>(x_dev), xh, xl, M * d.d_model, s);
    });
    if (r) return r;
    g.A = xh; g.A2 = xl;
  } else {
    g.A = static_cast<const uint16_t*>(x_dev);
  }
  g.lda = d.d_model;
  const PackedMat mats[6] = {Ly.wq, Ly.wk, Ly.wv, Ly.fa, Ly.ga, Ly.wbeta};
  const int rows[6] = {m->Kq, m->Kq, m->V, d.rank_f, d.rank_g, d.n_heads};
  int first = 0;
  for (int i = 0; i < 6; ++i) {
    g.seg_b[i] = reinterpret_cast<const uint16_t*>(mats[i].w);
    g.seg_first[i] = first;
    first += rows[i];
  }
  g.nseg = 6; g.M = (int)M; g.N = m->proj_rows; g.K = d.d_model;
  g.C = F(wl.P); g.ldc = m->proj_stride; g.coff = 0;
  r = timed(m, KDA_K_GEMM, s, rec, [&] { return launch_gemm(g, s); });
  if (r) return r;
  PrefillParams p;
  p.B = B; p.L = (int)L; p.H = d.n_heads; p.dk = d.d_k; p.dv = d.d_v; p.C = m->C;
  p.rank_f = d.rank_f; p.rank_g = d.rank_g;
  p.nch = (int)((L + kChunk - 1) / kChunk);
  p.P = F(wl.P); p.proj_stride = m->proj_stride;
  p.win = st->conv_dev; p.win_out = st->conv_dev;
  p.conv_w = Ly.conv_w; p.a_log = Ly.a_log; p.dt_bias = Ly.dt_bias; p.onw = Ly.o_norm_w;
  p.Fb = reinterpret_cast<const uint16_t*>(Ly.fb.w);
  p.gate = d.gate; p.gate_lb = d.gate_lb;
  p.Gb = reinterpret_cast<const uint16_t*>(Ly.gb.w);
  p.l2_eps = d.l2_eps; p.q_scale = m->q_scale; p.norm_eps = d.norm_eps;
  p.Wf = F(wl.W); p.Uf = F(wl.U); p.Qf = F(wl.Qt); p.Kf = F(wl.Kt); p.Af = F(wl.A); p.dec = F(wl.dec);
  p.S = st->S_dev; p.o = F(wl.o);
  p.on_hi = U16(wl.on); p.on_lo = p.on_hi + (size_t)M * m->V;
  // P2 / P3: conv + SiLU, norms, gates and the WY/UT form per chunk; the final window
  // (after the preparation, which reads the initial one); P4: the scan over chunks
  r = timed(m, KDA_K_CHUNK, s, rec, [&] { return launch_chunk_prep(p, s); });
  if (r) return r;
  r = timed(m, KDA_K_PREFILL, s, rec, [&] { return launch_prefill_window(p, s); });
  if (r) return r;
  r = timed(m, KDA_K_CHUNK, s, rec, [&] { return launch_chunk_scan(p, s); });
  if (r) return r;
  // P5: gated RMSNorm (as BF16 hi/lo planes), then the output projection over both planes
  r = timed(m, KDA_K_PREFILL, s, rec, [&] { return launch_chunk_gnorm(p, s); });
  if (r) return r;
  GemmParams go;
  go.A = p.on_hi; go.A2 = p.on_lo; go.lda = m->V;
  go.seg_b[0] = reinterpret_cast<const uint16_t*>(Ly.wo.w); go.nseg = 1;
  go.M = (int)M; go.N = d.d_model; go.K = m->V;
  go.C = y_dev; go.ldc = d.d_model; go.coff = 0;
  return timed(m, KDA_K_GEMM, s, rec, [&] { return launch_gemm(go, s); });
}

}  // extern "C"
