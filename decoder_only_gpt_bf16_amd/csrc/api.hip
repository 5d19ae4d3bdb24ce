// C ABI of the library (declared in include/gptmi.h): argument validation,
// saved-activation and workspace planning, and the launch sequence of each
// entry point on the caller's stream.  No allocation, no synchronisation.
#include <cmath>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gptmi.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIPCHK(call)                                                                       \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) return fail(GPT_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)

// Optional per-call-site timing: a pair of events recorded on the call's
// stream around each kernel call site, from a pool created by
// gpt_trace_begin (diagnostics only; off by default).
struct TraceState {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<std::pair<const char*, size_t>> recs;  // name, first event index
} g_trace;

struct TraceScope {
  hipStream_t s;
  const char* name;
  long idx = -1;
  TraceScope(const char* n, hipStream_t st) : s(st), name(n) {
    if (!g_trace.on) return;
    std::lock_guard<std::mutex> lk(g_trace.mu);
    if (g_trace.used + 2 > g_trace.pool.size()) return;
    idx = (long)g_trace.used;
    g_trace.used += 2;
    (void)hipEventRecord(g_trace.pool[idx], s);
  }
  ~TraceScope() {
    if (idx < 0) return;
    std::lock_guard<std::mutex> lk(g_trace.mu);
    (void)hipEventRecord(g_trace.pool[idx + 1], s);
    g_trace.recs.emplace_back(name, (size_t)idx);
  }
};

// Launch a kernel call site under a name (timed when tracing is on).
#define RUN(name, call)                  \
  do {                                   \
    TraceScope ts_(name, s);             \
    HIPCHK(call);                        \
  } while (0)

// Sequential 256-byte aligned carving of a buffer; with base == nullptr it
// only measures.
struct Arena {
  char* base;
  size_t off = 0;
  explicit Arena(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    off = align256(off);
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
  template <typename T> T* take_n(size_t n) { return static_cast<T*>(take(n * sizeof(T))); }
  size_t used() const { return align256(off); }
};

struct Dims {
  int B, T, N, C, H, D, V, dtype;
  size_t es;  // storage element size
};

constexpr long MAX_OPERAND_BYTES = 1L << 31;

int check_cfg(const gpt_config* cfg, Dims& d) {
  if (!cfg) return fail(GPT_ERR_INVALID, "cfg is NULL");
  if (cfg->n_head <= 0 || cfg->n_embd <= 0 || cfg->block_size <= 0 || cfg->vocab_size <= 0)
    return fail(GPT_ERR_INVALID, "non-positive n_head/n_embd/block_size/vocab_size");
  if (cfg->n_embd % cfg->n_head) return fail(GPT_ERR_INVALID, "n_embd %% n_head != 0");
  if (cfg->dtype != GPT_DTYPE_FP32 && cfg->dtype != GPT_DTYPE_BF16)
    return fail(GPT_ERR_UNSUPPORTED, "unknown dtype %d", cfg->dtype);
  if (cfg->norm != GPT_NORM_LAYERNORM && cfg->norm != GPT_NORM_RMSNORM)
    return fail(GPT_ERR_INVALID, "unknown norm %d", cfg->norm);
  if (!(cfg->norm_eps >= 0.0f)) return fail(GPT_ERR_INVALID, "norm_eps must be >= 0");
  if (cfg->attn_window < 0) return fail(GPT_ERR_INVALID, "attn_window must be >= 0");
  d.C = cfg->n_embd;
  d.H = cfg->n_head;
  d.D = d.C / d.H;
  d.V = cfg->vocab_size;
  d.dtype = cfg->dtype;
  d.es = cfg->dtype == GPT_DTYPE_BF16 ? 2 : 4;
  if (cfg->rope && (d.D & 1)) return fail(GPT_ERR_INVALID, "odd head_dim %d with rope", d.D);
  if (cfg->rope && !(cfg->rope_base > 0.0f)) return fail(GPT_ERR_INVALID, "rope_base must be > 0");
  if (d.D % 8 || d.D > 128) return fail(GPT_ERR_UNSUPPORTED, "head_dim %d not a multiple of 8 in [8, 128]", d.D);
  if (cfg->fp8 && (cfg->dtype != GPT_DTYPE_BF16 || d.C % 16))
    return fail(GPT_ERR_UNSUPPORTED, "fp8 needs bf16 storage and n_embd %% 16 == 0");
  if (d.C > 2048) return fail(GPT_ERR_UNSUPPORTED, "n_embd %d > 2048", d.C);
  return GPT_OK;
}

int check_bt(const gpt_config* cfg, int B, int T, Dims& d) {
  int st = check_cfg(cfg, d);
  if (st) return st;
  if (B <= 0 || T <= 0) return fail(GPT_ERR_INVALID, "B and T must be positive (B=%d T=%d)", B, T);
  if (T > cfg->block_size) return fail(GPT_ERR_INVALID, "T=%d exceeds block_size=%d", T, cfg->block_size);
  // the kernels address their operands through buffer descriptors with
  // 31-bit byte offsets: the largest one, [B*T, 4C] (GELU(u), GELU'(u), du),
  // must stay below 2 GiB, so larger batches are refused before any launch
  if ((long)B * T * 4L * cfg->n_embd * (long)d.es >= MAX_OPERAND_BYTES)
    return fail(GPT_ERR_UNSUPPORTED, "B*T*4*n_embd = %ld elements: an operand of 2 GiB or more", (long)B * T * 4L * cfg->n_embd);
  d.B = B;
  d.T = T;
  d.N = B * T;
  return GPT_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// ------------------------------------------------------------ block layouts
struct Saved {
  float2* cs;                            // RoPE (cos, sin) table [T][D/2], written by the forward
  void *a1, *qkv, *o, *x1, *a2, *u, *g;  // u holds GELU'(fc output), g = GELU(fc output)
  float *stats1, *stats2, *qkr, *lse;
  // FP8 (cfg->fp8): per-tensor quantizer scales [8][4] of a1, W_qkv, o, W_o,
  // a2, W_fc, g, W_proj; transposed codes of those activations [In][Np] and
  // weights [In][Out] for the backward's GEMMs
  float* f8sc;
  uint8_t *qa1T, *qoT, *qa2T, *qgT, *qWqkvT, *qWoT, *qWfcT, *qWprojT;
  // bf16 GEMMs: transposed copies of W_fc [C][4C], W_o [C][C] and W_qkv
  // [C][3C], written by the forward, read by the backward's input gradients
  void *wt_fc, *wt_o, *wt_qkv;
};
// the bf16 (non-FP8) block keeps transposed weights in `saved`
bool keeps_wt(const Dims& d, const gpt_config* cfg) { return d.dtype == GPT_DTYPE_BF16 && !cfg->fp8; }

// tokens padded to whole 64-row tiles of the transposed codes
long fp8_np(long N) { return (N + 63) / 64 * 64; }
long fp8_ld64(long n) { return (n + 63) / 64 * 64; }

Saved saved_layout(const Dims& d, const gpt_config* cfg, Arena& a) {
  Saved s{};
  const size_t N = d.N, C = d.C, es = d.es;
  s.cs = cfg->rope ? a.take_n<float2>((size_t)d.T * (d.D / 2)) : nullptr;
  s.a1 = a.take(N * C * es);
  s.stats1 = a.take_n<float>(2 * N);
  s.qkv = a.take(N * 3 * C * es);
  s.qkr = cfg->qk_norm ? a.take_n<float>(2 * N * d.H) : nullptr;
  s.o = a.take(N * C * es);
  s.lse = a.take_n<float>((size_t)d.B * d.H * d.T);
  s.x1 = a.take(N * C * es);
  s.a2 = a.take(N * C * es);
  s.stats2 = a.take_n<float>(2 * N);
  s.u = a.take(N * 4 * C * es);
  s.g = a.take(N * 4 * C * es);
  if (cfg->fp8) {
    const size_t Np = fp8_np(N);
    s.f8sc = a.take_n<float>(32);
    s.qa1T = a.take_n<uint8_t>(C * Np);
    s.qoT = a.take_n<uint8_t>(C * Np);
    s.qa2T = a.take_n<uint8_t>(C * Np);
    s.qgT = a.take_n<uint8_t>(4 * C * Np);
    s.qWqkvT = a.take_n<uint8_t>(C * fp8_ld64(3 * C));
    s.qWoT = a.take_n<uint8_t>(C * fp8_ld64(C));
    s.qWfcT = a.take_n<uint8_t>(C * fp8_ld64(4 * C));
    s.qWprojT = a.take_n<uint8_t>(4 * C * fp8_ld64(C));
  }
  if (keeps_wt(d, cfg)) {
    s.wt_fc = a.take(4 * C * C * es);
    s.wt_o = a.take(C * C * es);
    s.wt_qkv = a.take(3 * C * C * es);
  }
  return s;
}

// FP8 forward temporaries: codes of the current Linear's activation, of the
// four weights (qkv, o, fc, proj), amax partials
struct Fp8FwdWs {
  uint8_t* qx;
  uint8_t* qw[4];
  float* part;
};
Fp8FwdWs fp8_fwd_layout(const Dims& d, Arena& a) {
  Fp8FwdWs f{};
  const size_t N = d.N, C = d.C;
  f.qx = a.take_n<uint8_t>(N * 4 * C);
  f.qw[0] = a.take_n<uint8_t>(3 * C * C);
  f.qw[1] = a.take_n<uint8_t>(C * C);
  f.qw[2] = a.take_n<uint8_t>(4 * C * C);
  f.qw[3] = a.take_n<uint8_t>(4 * C * C);
  f.part = a.take_n<float>(fp8_q2d_parts(4));
  return f;
}

struct BwdWs {
  void *du, *da, *dx1, *dO, *dqkv;
  float *delta, *split;
  // column partials, each reduction its own so that one launch at the end
  // finishes them all: the two LayerNorms' gain and bias [2][nblk][C], the
  // biases of proj, fc, out and qkv [colsum_part_blocks(N)][width]
  float *colpart1, *colpart2, *bpart[4];
  // FP8: codes of the current gradient [N][Out]; each gradient's transposed
  // codes [Out][Np] (dy, du, dx1, dqkv), kept for the grouped weight
  // gradients at the end; amax partials, the gradients' scales [4][4]
  uint8_t *qg, *qgT[4];
  float *f8part, *f8sc;
};

GemmDesc gemm0() {
  GemmDesc g;
  memset(&g, 0, sizeof g);
  return g;
}

// forward Linear: out[N, Nout] = act[N, K] W[Nout, K]^T
GemmDesc lin_fwd(const Dims& d, const void* act, int K, const void* W, int Nout, int epi) {
  GemmDesc g = gemm0();
  g.A = act; g.lda = K; g.a_kmaj = false;
  g.B = W; g.ldb = K; g.b_kmaj = false;
  g.M = d.N; g.N = Nout; g.K = K; g.epi = epi;
  return g;
}
// input gradient: dX[N, In] = dY[N, Out] W[Out, In]
GemmDesc lin_dgrad(const Dims& d, const void* dY, int Out, const void* W, int In, int epi) {
  GemmDesc g = gemm0();
  g.A = dY; g.lda = Out; g.a_kmaj = false;
  g.B = W; g.ldb = In; g.b_kmaj = true;
  g.M = d.N; g.N = In; g.K = Out; g.epi = epi;
  return g;
}
// the same from a transposed copy WT[In, Out] of the weight: both operands
// then have k contiguous
GemmDesc lin_dgrad_t(const Dims& d, const void* dY, int Out, const void* WT, int In, int epi) {
  GemmDesc g = gemm0();
  g.A = dY; g.lda = Out; g.a_kmaj = false;
  g.B = WT; g.ldb = Out; g.b_kmaj = false;
  g.M = d.N; g.N = In; g.K = Out; g.epi = epi;
  return g;
}
// weight gradient: dW[Out, In] (+)= dY[N, Out]^T X[N, In]
GemmDesc lin_wgrad(const Dims& d, const void* dY, int Out, const void* X, int In, float* dW, int accumulate) {
  GemmDesc g = gemm0();
  g.A = dY; g.lda = Out; g.a_kmaj = true;
  g.B = X; g.ldb = In; g.b_kmaj = true;
  g.M = Out; g.N = In; g.K = d.N; g.epi = EPI_F32;
  g.out = dW; g.ldc = In; g.accumulate = accumulate;
  return g;
}

// the block's four weight gradients, in the order the backward forms them
void block_wgrads(const Dims& d, GemmDesc* wg) {
  const int C = d.C;
  wg[0] = lin_wgrad(d, nullptr, C, nullptr, 4 * C, nullptr, 0);   // proj
  wg[1] = lin_wgrad(d, nullptr, 4 * C, nullptr, C, nullptr, 0);   // fc
  wg[2] = lin_wgrad(d, nullptr, C, nullptr, C, nullptr, 0);       // out
  wg[3] = lin_wgrad(d, nullptr, 3 * C, nullptr, C, nullptr, 0);   // qkv
}

// FP8 weight gradient dW[Out, In] = q(dY)^T q(X): both operands transposed
// codes [.][Np], k = tokens
GemmDesc fp8_wgrad(const Dims& d, const void* qdyT, int Out, const void* qxT, int In, float* dW, int accumulate) {
  GemmDesc g = gemm0();
  const long Np = fp8_np(d.N);
  g.A = qdyT; g.lda = Np; g.B = qxT; g.ldb = Np;
  g.M = Out; g.N = In; g.K = (int)Np; g.epi = EPI_F32;
  g.out = dW; g.ldc = In; g.accumulate = accumulate;
  return g;
}

size_t split_need(const Dims& d, const gpt_config* cfg) {
  GemmDesc wg[4];
  block_wgrads(d, wg);
  size_t need = gemm_group_scratch_bytes(wg, 4, d.dtype);
  if (cfg->fp8) {
    // the grouped FP8 weight gradients, in the backward's order
    const int C = d.C;
    const GemmDesc f[4] = {fp8_wgrad(d, nullptr, C, nullptr, 4 * C, nullptr, 0),
                           fp8_wgrad(d, nullptr, 4 * C, nullptr, C, nullptr, 0),
                           fp8_wgrad(d, nullptr, C, nullptr, C, nullptr, 0),
                           fp8_wgrad(d, nullptr, 3 * C, nullptr, C, nullptr, 0)};
    need = std::max(need, gemm_group_fp8_scratch_bytes(f, 4));
  }
  return need;
}

BwdWs bwd_layout(const Dims& d, const gpt_config* cfg, Arena& a) {
  BwdWs w{};
  const size_t N = d.N, C = d.C, es = d.es;
  w.du = a.take(N * 4 * C * es);
  w.da = a.take(N * C * es);
  w.dx1 = a.take(N * C * es);
  w.dO = a.take(N * C * es);
  w.dqkv = a.take(N * 3 * C * es);
  w.delta = a.take_n<float>((size_t)d.B * d.H * d.T);
  if (cfg->norm == GPT_NORM_LAYERNORM) {
    w.colpart1 = a.take_n<float>(2 * (size_t)norm_bwd_blocks(d.N) * C);
    w.colpart2 = a.take_n<float>(2 * (size_t)norm_bwd_blocks(d.N) * C);
  }
  if (cfg->bias) {
    const int widths[4] = {(int)C, 4 * (int)C, (int)C, 3 * (int)C};
    for (int i = 0; i < 4; ++i) w.bpart[i] = static_cast<float*>(a.take(colsum_scratch_bytes(d.N, widths[i])));
  }
  w.split = static_cast<float*>(a.take(split_need(d, cfg)));
  if (cfg->fp8) {
    w.qg = a.take_n<uint8_t>(N * 4 * C);
    const size_t outs[4] = {C, 4 * C, C, 3 * C};
    for (int i = 0; i < 4; ++i) w.qgT[i] = a.take_n<uint8_t>(outs[i] * fp8_np(N));
    w.f8part = a.take_n<float>(fp8_q2d_parts(1));
    w.f8sc = a.take_n<float>(16);
  }
  return w;
}

size_t fwd_ws_bytes(const Dims& d, const gpt_config* cfg, bool inference) {
  Arena a(nullptr);
  if (inference) saved_layout(d, cfg, a);
  if (cfg->fp8) fp8_fwd_layout(d, a);
  return a.used();
}

// ------------------------------------------------------------ LM head layout
struct XentWs {
  int Vc, nchunk, P;
  long ldz;
  float2* part;
  float *ztgt, *lse, *nats, *loss_part, *dh_acc, *zbuf, *split;
  float2* run;
  void* dz;
};

constexpr int XENT_CHUNK = 8192;

XentWs xent_layout(const Dims& d, int N, Arena& a) {
  XentWs x{};
  const int V = d.V;
  x.Vc = std::min(V, XENT_CHUNK);
  x.nchunk = cdiv(V, x.Vc);
  x.ldz = (x.Vc + 7) / 8 * 8;
  int P = 0;
  for (int c = 0; c < x.nchunk; ++c) {
    const int w = std::min(x.Vc, V - c * x.Vc);
    P += (256 / xent_part_cols()) * cdiv(w, 256);
  }
  x.P = P;
  const bool mfma = d.dtype == 1;
  x.part = mfma ? a.take_n<float2>((size_t)N * P) : nullptr;
  x.run = mfma ? nullptr : a.take_n<float2>((size_t)N);
  x.ztgt = a.take_n<float>(N);
  x.lse = a.take_n<float>(N);
  x.nats = a.take_n<float>(N);
  x.loss_part = a.take_n<float>(xent_finish_blocks(N));
  x.dz = a.take((size_t)N * x.ldz * d.es);
  x.zbuf = mfma ? nullptr : a.take_n<float>((size_t)N * x.ldz);
  x.dh_acc = a.take_n<float>((size_t)N * d.C);
  size_t split = 0;
  for (int c = 0; c < x.nchunk; ++c) {
    const int w = std::min(x.Vc, V - c * x.Vc);
    GemmDesc g = gemm0();  // dW chunk = dz^T h
    g.M = w; g.N = d.C; g.K = N; g.epi = EPI_F32; g.a_kmaj = true; g.b_kmaj = true;
    GemmDesc q = gemm0();  // dh += dz W_chunk
    q.M = N; q.N = d.C; q.K = w; q.epi = EPI_F32; q.b_kmaj = true;
    split = std::max(split, std::max(gemm_split_scratch_bytes(g, d.dtype), gemm_split_scratch_bytes(q, d.dtype)));
  }
  x.split = static_cast<float*>(a.take(split));
  return x;
}

size_t xent_ws_bytes(const Dims& d, int N) {
  Arena a(nullptr);
  xent_layout(d, N, a);
  return a.used();
}

size_t embed_ws_bytes(const Dims& d) { return align256(embed_bwd_scratch_bytes(d.N, d.V)); }

size_t norm_ws_bytes(const Dims& d) { return align256(2 * (size_t)norm_bwd_blocks(d.N) * d.C * sizeof(float)); }

int check_block_weights(const gpt_config* cfg, const gpt_block_weights* w) {
  if (!w) return fail(GPT_ERR_INVALID, "weights struct is NULL");
  if (!w->w_qkv || !w->w_o || !w->w_fc || !w->w_proj) return fail(GPT_ERR_INVALID, "a Linear weight is NULL");
  if (cfg->norm == GPT_NORM_LAYERNORM && (!w->ln1_w || !w->ln2_w))
    return fail(GPT_ERR_INVALID, "LayerNorm gain is NULL");
  if (cfg->bias) {
    if (!w->b_qkv || !w->b_o || !w->b_fc || !w->b_proj) return fail(GPT_ERR_INVALID, "a Linear bias is NULL");
    if (cfg->norm == GPT_NORM_LAYERNORM && (!w->ln1_b || !w->ln2_b))
      return fail(GPT_ERR_INVALID, "LayerNorm bias is NULL");
  }
  const void* ps[] = {w->ln1_w, w->ln1_b, w->w_qkv, w->b_qkv, w->w_o, w->b_o,
                      w->ln2_w, w->ln2_b, w->w_fc, w->b_fc, w->w_proj, w->b_proj};
  for (const void* p : ps)
    if (p && !aligned16(p)) return fail(GPT_ERR_INVALID, "weight pointer not 16-byte aligned");
  return GPT_OK;
}

const void* opt(const gpt_config* cfg, const void* p) { return cfg->bias ? p : nullptr; }

}  // namespace

extern "C" {

const char* gpt_status_string(int status) {
  switch (status) {
    case GPT_OK: return "ok";
    case GPT_ERR_INVALID: return "invalid argument";
    case GPT_ERR_UNSUPPORTED: return "unsupported configuration";
    case GPT_ERR_WORKSPACE: return "workspace too small";
    case GPT_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* gpt_last_error(void) { return g_err.c_str(); }

int gpt_trace_begin(int capacity) {
  if (capacity <= 0) return fail(GPT_ERR_INVALID, "capacity must be positive");
  std::lock_guard<std::mutex> lk(g_trace.mu);
  while (g_trace.pool.size() < 2 * (size_t)capacity) {
    hipEvent_t e;
    HIPCHK(hipEventCreate(&e));
    g_trace.pool.push_back(e);
  }
  g_trace.used = 0;
  g_trace.recs.clear();
  g_trace.on = true;
  return GPT_OK;
}

int gpt_trace_end(char* buf, size_t len) {
  std::lock_guard<std::mutex> lk(g_trace.mu);
  g_trace.on = false;
  std::map<std::string, std::pair<long, double>> agg;
  std::vector<std::string> order;
  for (auto& r : g_trace.recs) {
    HIPCHK(hipEventSynchronize(g_trace.pool[r.second + 1]));
    float ms = 0.0f;
    HIPCHK(hipEventElapsedTime(&ms, g_trace.pool[r.second], g_trace.pool[r.second + 1]));
    auto it = agg.find(r.first);
    if (it == agg.end()) { order.push_back(r.first); agg[r.first] = {1, ms * 1000.0}; }
    else { it->second.first += 1; it->second.second += ms * 1000.0; }
  }
  std::string out;
  char line[160];
  for (auto& n : order) {
    snprintf(line, sizeof line, "%s %ld %.3f\n", n.c_str(), agg[n].first, agg[n].second);
    out += line;
  }
  g_trace.recs.clear();
  g_trace.used = 0;
  if (buf && len) {
    strncpy(buf, out.c_str(), len - 1);
    buf[len - 1] = 0;
  }
  if (out.size() + 1 > len) return fail(GPT_ERR_INVALID, "trace buffer too small (%zu bytes needed)", out.size() + 1);
  return GPT_OK;
}

size_t gpt_block_saved_bytes(const gpt_config* cfg, int B, int T) {
  Dims d;
  if (check_bt(cfg, B, T, d)) return 0;
  Arena a(nullptr);
  saved_layout(d, cfg, a);
  return a.used();
}

size_t gpt_workspace_bytes(const gpt_config* cfg, int B, int T) {
  Dims d;
  if (check_bt(cfg, B, T, d)) return 0;
  size_t m = fwd_ws_bytes(d, cfg, true);
  Arena a(nullptr);
  bwd_layout(d, cfg, a);
  m = std::max(m, a.used());
  m = std::max(m, xent_ws_bytes(d, d.N));
  m = std::max(m, embed_ws_bytes(d));
  m = std::max(m, norm_ws_bytes(d));
  return m;
}

int gpt_block_fwd(const gpt_config* cfg, int B, int T, const void* x, const gpt_block_weights* w, void* y,
                  void* saved, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_bt(cfg, B, T, d);
  if (st) return st;
  if ((st = check_block_weights(cfg, w))) return st;
  if (!x || !y) return fail(GPT_ERR_INVALID, "x or y is NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(saved) || !aligned16(ws))
    return fail(GPT_ERR_INVALID, "buffer not 16-byte aligned");
  const size_t need = fwd_ws_bytes(d, cfg, saved == nullptr);
  if (need && (!ws || ws_bytes < need))
    return fail(GPT_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  Arena sa(saved ? saved : ws);  // inference: intermediates live in the workspace
  Saved sv = saved_layout(d, cfg, sa);
  float2* cs = sv.cs;
  const int C = d.C, ty = d.dtype, kind = cfg->norm;
  Arena fa = saved ? Arena(ws) : sa;  // FP8 temporaries follow the intermediates
  const Fp8FwdWs fw = cfg->fp8 ? fp8_fwd_layout(d, fa) : Fp8FwdWs{};

  // FP8: the four weights quantized to E4M3 in one pass (codes for the
  // forward GEMMs, transposed codes kept in `saved` for the backward's)
  if (cfg->fp8) {
    const Fp8Q2d qw[4] = {
        {w->w_qkv, fw.qw[0], saved ? sv.qWqkvT : nullptr, fp8_ld64(3 * C), 3 * C, C, sv.f8sc + 4 * 1},
        {w->w_o, fw.qw[1], saved ? sv.qWoT : nullptr, fp8_ld64(C), C, C, sv.f8sc + 4 * 3},
        {w->w_fc, fw.qw[2], saved ? sv.qWfcT : nullptr, fp8_ld64(4 * C), 4 * C, C, sv.f8sc + 4 * 5},
        {w->w_proj, fw.qw[3], saved ? sv.qWprojT : nullptr, fp8_ld64(C), C, 4 * C, sv.f8sc + 4 * 7}};
    RUN("fp8_quant_w", launch_fp8_quantize_2d(qw, 4, FP8_E4M3, fw.part, s));
  }
  // One Linear layer: the bf16 GEMM, or with cfg->fp8 the activation
  // quantized to E4M3 (its transposed codes kept in `saved` for the
  // backward) and the FP8 GEMM with the same epilogue.  slot: the
  // activation's scale slot in sv.f8sc, the weight's is slot + 1; wi: the
  // weight's codes in fw.qw.
  auto linear = [&](const char* name, GemmDesc g, int slot, uint8_t* qxT, int wi) -> int {
    if (!cfg->fp8) {
      RUN(name, launch_gemm(g, ty, nullptr, s));
      return GPT_OK;
    }
    const int In = g.K;
    float* sx = sv.f8sc + 4 * slot;
    const Fp8Q2d qx = {g.A, fw.qx, saved ? qxT : nullptr, fp8_np(d.N), d.N, In, sx};
    RUN("fp8_quant_x", launch_fp8_quantize_2d(&qx, 1, FP8_E4M3, fw.part, s));
    g.A = fw.qx; g.lda = In; g.B = fw.qw[wi]; g.ldb = In;
    g.f8_sa = sx; g.f8_sb = sv.f8sc + 4 * (slot + 1);
    RUN(name, launch_gemm_fp8(g, 1, nullptr, s));
    return GPT_OK;
  };

  // norm1's launch also writes the RoPE table (positions 0..T-1) for the
  // QKV epilogue and the backward; theta_i = base^(-2i/D) in double
  RopeJob rope{};
  if (cfg->rope) {
    rope.cs = cs;
    rope.T = T;
    rope.half = d.D / 2;
    for (int i = 0; i < rope.half; ++i) rope.theta[i] = std::pow((double)cfg->rope_base, -2.0 * i / d.D);
  }
  RUN("norm1_fwd", launch_norm_fwd(ty, kind, d.N, C, x, w->ln1_w, opt(cfg, w->ln1_b), cfg->norm_eps, sv.a1, sv.stats1, s,
                                   &rope));
  // RoPE / QK-norm ride in the QKV GEMM's epilogue when a wave's 128 output
  // columns are exactly one head (bf16, head_dim 128); else a separate pass
  const bool qk = cfg->rope || cfg->qk_norm;
  const bool qk_fused = qk && ty == GPT_DTYPE_BF16 && d.D == 128;
  GemmDesc g = lin_fwd(d, sv.a1, C, w->w_qkv, 3 * C, qk_fused ? EPI_QKNORM : EPI_STORE);
  g.out = sv.qkv; g.ldc = 3 * C; g.bias = opt(cfg, w->b_qkv);
  if (qk_fused) {
    g.qk_cs = cs; g.qk_rstd = sv.qkr; g.qk_T = T; g.qk_rope = cfg->rope; g.qk_norm = cfg->qk_norm;
    g.qk_eps = cfg->norm_eps;
  }
  if ((st = linear("qkv_gemm", g, 0, sv.qa1T, 0))) return st;
  if (qk && !qk_fused)
    RUN("qk_rope_norm", launch_qk_fwd(ty, B, T, d.H, d.D, cfg->rope, cfg->qk_norm, cfg->norm_eps, cs, sv.qkv, sv.qkr, s));
  // the backward's transposed weights ride in the attention launch, whose
  // tail has CUs to spare (training only: inference needs none)
  const bool wt = saved && keeps_wt(d, cfg);
  const TransposeDesc td[3] = {{w->w_fc, sv.wt_fc, 4 * C, C}, {w->w_o, sv.wt_o, C, C}, {w->w_qkv, sv.wt_qkv, 3 * C, C}};
  RUN("attn_fwd", launch_attn_fwd(ty, B, T, d.H, d.D, cfg->qk_norm, cfg->attn_window, sv.qkv, sv.o, sv.lse, td,
                                  wt ? 3 : 0, s));
  g = lin_fwd(d, sv.o, C, w->w_o, C, EPI_STORE);
  g.out = sv.x1; g.ldc = C; g.bias = opt(cfg, w->b_o); g.resid = x; g.ldr = C;
  if ((st = linear("out_gemm", g, 2, sv.qoT, 1))) return st;
  RUN("norm2_fwd", launch_norm_fwd(ty, kind, d.N, C, sv.x1, w->ln2_w, opt(cfg, w->ln2_b), cfg->norm_eps, sv.a2, sv.stats2, s));
  g = lin_fwd(d, sv.a2, C, w->w_fc, 4 * C, EPI_GELU);
  // inference keeps no GELU'(u): the epilogue then writes GELU(u) only
  g.out = saved ? sv.u : nullptr; g.out2 = sv.g; g.ldc = 4 * C; g.bias = opt(cfg, w->b_fc);
  if ((st = linear("fc_gemm_gelu", g, 4, sv.qa2T, 2))) return st;
  g = lin_fwd(d, sv.g, 4 * C, w->w_proj, C, EPI_STORE);
  g.out = y; g.ldc = C; g.bias = opt(cfg, w->b_proj); g.resid = sv.x1; g.ldr = C;
  if ((st = linear("proj_gemm", g, 6, sv.qgT, 3))) return st;
  return GPT_OK;
}

int gpt_block_bwd(const gpt_config* cfg, int B, int T, const void* x, const void* dy, const gpt_block_weights* w,
                  const void* saved, void* dx, const gpt_block_grads* gr, int accumulate, void* ws,
                  size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_bt(cfg, B, T, d);
  if (st) return st;
  if ((st = check_block_weights(cfg, w))) return st;
  if (!x || !dy || !saved || !dx || !gr) return fail(GPT_ERR_INVALID, "x, dy, saved, dx or grads is NULL");
  if (!gr->w_qkv || !gr->w_o || !gr->w_fc || !gr->w_proj) return fail(GPT_ERR_INVALID, "a weight gradient is NULL");
  if (cfg->norm == GPT_NORM_LAYERNORM && (!gr->ln1_w || !gr->ln2_w))
    return fail(GPT_ERR_INVALID, "LayerNorm gain gradient is NULL");
  if (cfg->bias && (!gr->b_qkv || !gr->b_o || !gr->b_fc || !gr->b_proj ||
                    (cfg->norm == GPT_NORM_LAYERNORM && (!gr->ln1_b || !gr->ln2_b))))
    return fail(GPT_ERR_INVALID, "a bias gradient is NULL");
  if (!aligned16(x) || !aligned16(dy) || !aligned16(saved) || !aligned16(dx) || !aligned16(ws))
    return fail(GPT_ERR_INVALID, "buffer not 16-byte aligned");
  Arena probe(nullptr);
  bwd_layout(d, cfg, probe);
  if (!ws || ws_bytes < probe.used())
    return fail(GPT_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, probe.used());
  hipStream_t s = static_cast<hipStream_t>(stream);
  Arena sa(const_cast<void*>(saved));
  Saved sv = saved_layout(d, cfg, sa);
  Arena wa(ws);
  BwdWs b = bwd_layout(d, cfg, wa);
  const int C = d.C, ty = d.dtype, kind = cfg->norm, N = d.N;
  const int nblk = norm_bwd_blocks(N);
  const bool ln = kind == GPT_NORM_LAYERNORM;

  // FP8 (cfg->fp8): each incoming gradient is quantized once (E5M2) into
  // codes for its input-gradient GEMM (the buffer serves the next layer)
  // and transposed codes of its own for the weight gradients, which run as
  // one grouped launch at the end as in bf16; the weights' and activations'
  // codes come from the forward.  Gradient slots (scales in b.f8sc,
  // transposed codes in b.qgT): 0 dy, 1 du, 2 dx1, 3 dqkv.
  const bool f8 = cfg->fp8 != 0;
  auto fp8_grad = [&](const void* dY, int Out, int slot) -> int {
    const Fp8Q2d qg = {dY, b.qg, b.qgT[slot], fp8_np(N), N, Out, b.f8sc + 4 * slot};
    RUN("fp8_quant_g", launch_fp8_quantize_2d(&qg, 1, FP8_E5M2, b.f8part, s));
    return GPT_OK;
  };
  // dX[N][In] = q(dY) q(W): the forward's transposed weight codes [In][ld64(Out)]
  auto fp8_dgrad = [&](const char* name, GemmDesc g, int Out, const uint8_t* qWT, int In, int gslot,
                       int wslot) -> int {
    g.A = b.qg; g.lda = Out; g.a_kmaj = false;
    g.B = qWT; g.ldb = fp8_ld64(Out); g.b_kmaj = false;
    g.M = N; g.N = In; g.K = Out;
    g.f8_sa = b.f8sc + 4 * gslot; g.f8_sb = sv.f8sc + 4 * wslot;
    RUN(name, launch_gemm_fp8(g, 2, nullptr, s));
    return GPT_OK;
  };
  // dW[Out][In] (+)= q(dY)^T q(X): the gradient's and the activation's
  // transposed codes, gathered for the grouped launch at the end
  GemmDesc wg8[GEMM_GROUP_MAX];
  int nwg8 = 0;
  auto fp8_wg = [&](int Out, const uint8_t* qxT, int In, float* dW, int gslot, int xslot) {
    GemmDesc g = fp8_wgrad(d, b.qgT[gslot], Out, qxT, In, dW, accumulate);
    g.f8_sa = b.f8sc + 4 * gslot; g.f8_sb = sv.f8sc + 4 * xslot;
    wg8[nwg8++] = g;
  };

  // bf16: the input gradients through W_fc, W_o and W_qkv read the
  // transposed copies the forward left in `saved` (k contiguous on both
  // sides of those GEMMs); W_proj's is read as it lies (its wide tiles run
  // as fast either way)
  const bool wt = keeps_wt(d, cfg);
  // weight gradients depend on nothing computed later: they are gathered
  // and run as one grouped launch at the end of the backward (one launch
  // fills the machine where each alone would leave CUs idle)
  GemmDesc wg[GEMM_GROUP_MAX];
  int nwg = 0;
  // MLP: y = x1 + gelu(a2 W_fc^T + b_fc) W_proj^T + b_proj
  GemmDesc g = lin_dgrad(d, dy, C, w->w_proj, 4 * C, EPI_GELU_BWD);
  g.out = b.du; g.ldc = 4 * C; g.aux = sv.u; g.ldaux = 4 * C;
  if (f8) {
    if ((st = fp8_grad(dy, C, 0))) return st;
    if ((st = fp8_dgrad("proj_dgrad_gelu", g, C, sv.qWprojT, 4 * C, 0, 7))) return st;
    fp8_wg(C, sv.qgT, 4 * C, gr->w_proj, 0, 6);
  } else {
    RUN("proj_dgrad_gelu", launch_gemm(g, ty, nullptr, s));
    wg[nwg++] = lin_wgrad(d, dy, C, sv.g, 4 * C, gr->w_proj, accumulate);
  }
  // column sums (bias and LayerNorm gradients): partials as their inputs
  // appear, one launch at the end reduces them all
  ColsumJob cj[COLSUM_JOBS_MAX];
  int ncj = 0;
  const int pb = colsum_part_blocks(N);
  if (cfg->bias) {
    RUN("proj_bias", launch_colsum_part(ty, N, C, C, dy, b.bpart[0], s));
    cj[ncj++] = {b.bpart[0], pb, C, gr->b_proj};
  }
  g = wt ? lin_dgrad_t(d, b.du, 4 * C, sv.wt_fc, C, EPI_STORE) : lin_dgrad(d, b.du, 4 * C, w->w_fc, C, EPI_STORE);
  g.out = b.da; g.ldc = C;
  if (f8) {
    if ((st = fp8_grad(b.du, 4 * C, 1))) return st;
    if ((st = fp8_dgrad("fc_dgrad", g, 4 * C, sv.qWfcT, C, 1, 5))) return st;
    fp8_wg(4 * C, sv.qa2T, C, gr->w_fc, 1, 4);
  } else {
    RUN("fc_dgrad", launch_gemm(g, ty, nullptr, s));
    wg[nwg++] = lin_wgrad(d, b.du, 4 * C, sv.a2, C, gr->w_fc, accumulate);
  }
  if (cfg->bias) {
    RUN("fc_bias", launch_colsum_part(ty, N, 4 * C, 4 * C, b.du, b.bpart[1], s));
    cj[ncj++] = {b.bpart[1], pb, 4 * C, gr->b_fc};
  }
  // norm 2 backward + residual
  RUN("norm2_bwd", launch_norm_bwd(ty, kind, N, C, sv.x1, w->ln2_w, b.da, dy, cfg->norm_eps, b.dx1, b.colpart2, ln, s));
  if (ln) {
    cj[ncj++] = {b.colpart2, nblk, C, gr->ln2_w};
    if (cfg->bias) cj[ncj++] = {b.colpart2 + (size_t)nblk * C, nblk, C, gr->ln2_b};
  }
  // attention output projection
  g = wt ? lin_dgrad_t(d, b.dx1, C, sv.wt_o, C, EPI_STORE) : lin_dgrad(d, b.dx1, C, w->w_o, C, EPI_STORE);
  g.out = b.dO; g.ldc = C;
  if (f8) {
    if ((st = fp8_grad(b.dx1, C, 2))) return st;
    if ((st = fp8_dgrad("out_dgrad", g, C, sv.qWoT, C, 2, 3))) return st;
    fp8_wg(C, sv.qoT, C, gr->w_o, 2, 2);
  } else {
    RUN("out_dgrad", launch_gemm(g, ty, nullptr, s));
    wg[nwg++] = lin_wgrad(d, b.dx1, C, sv.o, C, gr->w_o, accumulate);
  }
  if (cfg->bias) {
    RUN("out_bias", launch_colsum_part(ty, N, C, C, b.dx1, b.bpart[2], s));
    cj[ncj++] = {b.bpart[2], pb, C, gr->b_o};
  }
  // attention
  const QkBwd qk{cfg->rope, cfg->qk_norm, N, sv.cs, sv.qkr};
  if (attn_mfma_supported(ty, d.D)) {
    // dQ pass first (it also forms delta); QK-norm / RoPE backward in both stores
    RUN("attn_bwd_dq", launch_attn_bwd_dq(ty, B, T, d.H, d.D, cfg->attn_window, sv.qkv, sv.o, b.dO, sv.lse, b.delta,
                                          b.dqkv, qk, s));
    RUN("attn_bwd_dkdv", launch_attn_bwd_dkdv(ty, B, T, d.H, d.D, cfg->attn_window, sv.qkv, b.dO, sv.lse, b.delta,
                                              b.dqkv, qk, s));
  } else {
    RUN("attn_delta", launch_attn_delta(ty, B, T, d.H, d.D, sv.o, b.dO, b.delta, s));
    RUN("attn_bwd_dkdv", launch_attn_bwd_dkdv(ty, B, T, d.H, d.D, cfg->attn_window, sv.qkv, b.dO, sv.lse, b.delta,
                                              b.dqkv, qk, s));
    RUN("attn_bwd_dq", launch_attn_bwd_dq(ty, B, T, d.H, d.D, cfg->attn_window, sv.qkv, sv.o, b.dO, sv.lse, b.delta,
                                          b.dqkv, qk, s));
    if (cfg->rope || cfg->qk_norm)
      RUN("qk_bwd", launch_qk_bwd(ty, B, T, d.H, d.D, cfg->rope, cfg->qk_norm, sv.cs, sv.qkv, sv.qkr, b.dqkv, s));
  }
  // fused QKV projection
  g = wt ? lin_dgrad_t(d, b.dqkv, 3 * C, sv.wt_qkv, C, EPI_STORE)
         : lin_dgrad(d, b.dqkv, 3 * C, w->w_qkv, C, EPI_STORE);
  g.out = b.da; g.ldc = C;
  if (f8) {
    if ((st = fp8_grad(b.dqkv, 3 * C, 3))) return st;
    if ((st = fp8_dgrad("qkv_dgrad", g, 3 * C, sv.qWqkvT, C, 3, 1))) return st;
    fp8_wg(3 * C, sv.qa1T, C, gr->w_qkv, 3, 0);
  } else {
    RUN("qkv_dgrad", launch_gemm(g, ty, nullptr, s));
    wg[nwg++] = lin_wgrad(d, b.dqkv, 3 * C, sv.a1, C, gr->w_qkv, accumulate);
  }
  if (cfg->bias) {
    RUN("qkv_bias", launch_colsum_part(ty, N, 3 * C, 3 * C, b.dqkv, b.bpart[3], s));
    cj[ncj++] = {b.bpart[3], pb, 3 * C, gr->b_qkv};
  }
  // norm 1 backward + residual
  RUN("norm1_bwd", launch_norm_bwd(ty, kind, N, C, x, w->ln1_w, b.da, b.dx1, cfg->norm_eps, dx, b.colpart1, ln, s));
  if (ln) {
    cj[ncj++] = {b.colpart1, nblk, C, gr->ln1_w};
    if (cfg->bias) cj[ncj++] = {b.colpart1 + (size_t)nblk * C, nblk, C, gr->ln1_b};
  }
  if (nwg) RUN("wgrad_group", launch_gemm_group(wg, nwg, ty, b.split, split_need(d, cfg), s));
  if (nwg8) RUN("wgrad_group", launch_gemm_group_fp8(wg8, nwg8, b.split, split_need(d, cfg), s));
  if (ncj) RUN("col_sums", launch_colsum_finish_jobs(cj, ncj, accumulate, s));
  return GPT_OK;
}

static int xent_impl(const gpt_config* cfg, int N, const void* h, const void* W, const int32_t* targets,
                     const float* weight, float loss_scale, float* loss, float* nats, void* dh, float* dW,
                     int accumulate, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_cfg(cfg, d);
  if (st) return st;
  if (N <= 0) return fail(GPT_ERR_INVALID, "N must be positive");
  if (!h || !W || !targets || !loss) return fail(GPT_ERR_INVALID, "h, W, targets or loss is NULL");
  if (!aligned16(h) || !aligned16(W) || !aligned16(dh) || !aligned16(dW) || !aligned16(ws))
    return fail(GPT_ERR_INVALID, "buffer not 16-byte aligned");
  d.B = 1; d.T = N; d.N = N;
  {
    // the logit-gradient chunk [N, min(V, chunk)] and h [N, C] are GEMM
    // operands read through 31-bit buffer offsets
    const long ldz = (std::min(d.V, XENT_CHUNK) + 7) / 8 * 8;
    if ((long)N * std::max<long>(ldz, d.C) * (long)d.es >= MAX_OPERAND_BYTES)
      return fail(GPT_ERR_UNSUPPORTED, "N = %d: a logit chunk or h operand of 2 GiB or more", N);
  }
  const size_t need = xent_ws_bytes(d, N);
  if (!ws || ws_bytes < need) return fail(GPT_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  Arena wa(ws);
  XentWs x = xent_layout(d, N, wa);
  const int C = d.C, V = d.V, ty = d.dtype;
  float* nt = nats ? nats : x.nats;
  const bool mfma = ty == 1;
  // a target outside [0, V) matches no column: xent_finish gives it NaN nats
  for (int c = 0; c < x.nchunk; ++c) {
    const int v0 = c * x.Vc;
    const int Vw = std::min(x.Vc, V - v0);
    const void* Wc = static_cast<const char*>(W) + (size_t)v0 * C * d.es;
    GemmDesc g = gemm0();
    g.A = h; g.lda = C; g.B = Wc; g.ldb = C; g.M = N; g.N = Vw; g.K = C;
    if (mfma) {
      g.epi = EPI_XENT_STATS;
      g.tgt = targets; g.col_offset = v0; g.part = x.part; g.part_ld = x.P;
      int off = 0;
      for (int q = 0; q < c; ++q) off += (256 / xent_part_cols()) * cdiv(std::min(x.Vc, V - q * x.Vc), 256);
      g.part_off = off; g.ztgt = x.ztgt;
      RUN("xent_stats_gemm", launch_gemm(g, ty, nullptr, s));
    } else {
      g.epi = EPI_F32; g.out = x.zbuf; g.ldc = x.ldz;
      RUN("xent_logits_gemm", launch_gemm(g, ty, nullptr, s));
      RUN("xent_rows_stats", launch_xent_rows_stats(N, Vw, v0, x.zbuf, x.ldz, targets, x.run, x.ztgt, c == 0, s));
    }
  }
  RUN("xent_finish", launch_xent_finish(N, mfma ? x.P : 1, V, mfma ? x.part : x.run, targets, x.ztgt, weight, x.lse,
                                        nt, x.loss_part, s));
  RUN("loss_sum", launch_loss_sum(xent_finish_blocks(N), x.loss_part, loss_scale, loss, s));
  if (!dh && !dW) return GPT_OK;
  for (int c = 0; c < x.nchunk; ++c) {
    const int v0 = c * x.Vc;
    const int Vw = std::min(x.Vc, V - v0);
    const void* Wc = static_cast<const char*>(W) + (size_t)v0 * C * d.es;
    GemmDesc g = gemm0();
    g.A = h; g.lda = C; g.B = Wc; g.ldb = C; g.M = N; g.N = Vw; g.K = C;
    if (mfma) {
      g.epi = EPI_XENT_GRAD; g.out = x.dz; g.ldc = x.ldz;
      g.tgt = targets; g.col_offset = v0; g.lse = x.lse; g.scale = loss_scale; g.roww = weight;
      RUN("xent_grad_gemm", launch_gemm(g, ty, nullptr, s));
    } else {
      g.epi = EPI_F32; g.out = x.zbuf; g.ldc = x.ldz;
      RUN("xent_logits_gemm", launch_gemm(g, ty, nullptr, s));
      RUN("xent_rows_grad",
          launch_xent_rows_grad(ty, N, Vw, v0, x.zbuf, x.ldz, targets, x.lse, loss_scale, weight, x.dz, x.ldz, s));
    }
    if (dh) {
      GemmDesc q = gemm0();
      q.A = x.dz; q.lda = x.ldz; q.a_kmaj = false;
      q.B = Wc; q.ldb = C; q.b_kmaj = true;
      q.M = N; q.N = C; q.K = Vw; q.epi = EPI_F32; q.out = x.dh_acc; q.ldc = C; q.accumulate = c > 0;
      RUN("xent_dh_gemm", launch_gemm(q, ty, x.split, s));
    }
    if (dW) {
      GemmDesc q = gemm0();
      q.A = x.dz; q.lda = x.ldz; q.a_kmaj = true;
      q.B = h; q.ldb = C; q.b_kmaj = true;
      q.M = Vw; q.N = C; q.K = N; q.epi = EPI_F32; q.out = dW + (size_t)v0 * C; q.ldc = C;
      q.accumulate = accumulate;
      RUN("xent_dw_gemm", launch_gemm(q, ty, x.split, s));
    }
  }
  if (dh) RUN("xent_dh_convert", launch_f32_to(ty, (long)N * C, x.dh_acc, dh, s));
  return GPT_OK;
}

int lm_head_xent_fwd_bwd(const gpt_config* cfg, int N, const void* h, const void* W, const int32_t* targets,
                         float loss_scale, float* loss, float* nats, void* dh, float* dW, int accumulate, void* ws,
                         size_t ws_bytes, void* stream) {
  return xent_impl(cfg, N, h, W, targets, nullptr, loss_scale, loss, nats, dh, dW, accumulate, ws, ws_bytes, stream);
}

int lm_head_xent_weighted_fwd_bwd(const gpt_config* cfg, int N, const void* h, const void* W, const int32_t* targets,
                                  const float* token_weight, float loss_scale, float* loss, float* nats, void* dh,
                                  float* dW, int accumulate, void* ws, size_t ws_bytes, void* stream) {
  if (!token_weight) return fail(GPT_ERR_INVALID, "token_weight is NULL");
  return xent_impl(cfg, N, h, W, targets, token_weight, loss_scale, loss, nats, dh, dW, accumulate, ws, ws_bytes,
                   stream);
}

int val_bpb_reduce(int N, const float* nats, const int32_t* targets, const int32_t* token_bytes, int V,
                   double* sum_nats, int64_t* sum_bytes, void* stream) {
  if (N <= 0 || V <= 0) return fail(GPT_ERR_INVALID, "N and V must be positive");
  if (!nats || !targets || !token_bytes || !sum_nats || !sum_bytes)
    return fail(GPT_ERR_INVALID, "a pointer argument is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  RUN("bpb", launch_bpb(N, V, nats, targets, token_bytes, sum_nats, sum_bytes, s));
  return GPT_OK;
}

// ------------------------------------------------------------ FP8
size_t gpt_fp8_workspace_bytes(int64_t n) { return n > 0 ? align256((size_t)fp8_amax_parts(n) * sizeof(float)) : 0; }

int gpt_fp8_quantize(int64_t n, const void* x, int fmt, void* q, float* scale, void* ws, size_t ws_bytes,
                     void* stream) {
  if (n <= 0) return fail(GPT_ERR_INVALID, "n must be positive");
  if (fmt != GPT_FP8_E4M3 && fmt != GPT_FP8_E5M2) return fail(GPT_ERR_INVALID, "unknown fp8 format %d", fmt);
  if (!x || !q || !scale) return fail(GPT_ERR_INVALID, "x, q or scale is NULL");
  if (!aligned16(x) || !aligned16(q) || !aligned16(ws)) return fail(GPT_ERR_INVALID, "buffer not 16-byte aligned");
  const size_t need = gpt_fp8_workspace_bytes(n);
  if (!ws || ws_bytes < need) return fail(GPT_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, need);
  if (fp8_amax_parts(n) > (1L << 30)) return fail(GPT_ERR_INVALID, "n too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  RUN("fp8_quantize", launch_fp8_quantize((long)n, x, fmt, q, scale, static_cast<float*>(ws), s));
  return GPT_OK;
}

int gpt_fp8_gemm(int M, int N, int K, const void* qa, int64_t lda, int fmt_a, const float* scale_a, const void* qb,
                 int64_t ldb, int fmt_b, const float* scale_b, void* out, int64_t ldc, void* stream) {
  if (M <= 0 || N <= 0 || K <= 0) return fail(GPT_ERR_INVALID, "M, N and K must be positive");
  if ((fmt_a != GPT_FP8_E4M3 && fmt_a != GPT_FP8_E5M2) || (fmt_b != GPT_FP8_E4M3 && fmt_b != GPT_FP8_E5M2))
    return fail(GPT_ERR_INVALID, "unknown fp8 format");
  if (!qa || !qb || !scale_a || !scale_b || !out) return fail(GPT_ERR_INVALID, "a pointer argument is NULL");
  if (K % 16 || lda % 16 || ldb % 16 || lda < K || ldb < K)
    return fail(GPT_ERR_INVALID, "K, lda, ldb must be multiples of 16 with lda, ldb >= K");
  if (N % 8 || ldc % 8 || ldc < N) return fail(GPT_ERR_INVALID, "N and ldc must be multiples of 8 with ldc >= N");
  if (!aligned16(qa) || !aligned16(qb) || !aligned16(out)) return fail(GPT_ERR_INVALID, "buffer not 16-byte aligned");
  if ((M - 1) * lda + K >= (1L << 31) || (N - 1) * ldb + K >= (1L << 31))
    return fail(GPT_ERR_INVALID, "operand larger than 2 GiB");
  hipStream_t s = static_cast<hipStream_t>(stream);
  RUN("fp8_gemm", launch_fp8_gemm(M, N, K, qa, (long)lda, fmt_a, scale_a, qb, (long)ldb, fmt_b, scale_b, out,
                                  (long)ldc, s));
  return GPT_OK;
}

// ------------------------------------------------------------ optimizer
// The C descriptor and the kernels' one share their layout, so the caller's
// array is read in place (no copy, no allocation).
static_assert(sizeof(gpt_adamw_tensor) == sizeof(OptTensor), "descriptor layouts differ");
static_assert(offsetof(gpt_adamw_tensor, param) == offsetof(OptTensor, p), "descriptor layouts differ");
static_assert(offsetof(gpt_adamw_tensor, grad) == offsetof(OptTensor, g), "descriptor layouts differ");
static_assert(offsetof(gpt_adamw_tensor, m) == offsetof(OptTensor, m), "descriptor layouts differ");
static_assert(offsetof(gpt_adamw_tensor, v) == offsetof(OptTensor, v), "descriptor layouts differ");
static_assert(offsetof(gpt_adamw_tensor, param_bf16) == offsetof(OptTensor, p16), "descriptor layouts differ");
static_assert(offsetof(gpt_adamw_tensor, n) == offsetof(OptTensor, n), "descriptor layouts differ");
static_assert(offsetof(gpt_adamw_tensor, decay) == offsetof(OptTensor, decay), "descriptor layouts differ");

static int adamw_tensors(const gpt_adamw_tensor* tensors, int count, const OptTensor** out) {
  if (!tensors || count <= 0) return fail(GPT_ERR_INVALID, "no tensors");
  for (int i = 0; i < count; ++i) {
    const gpt_adamw_tensor& t = tensors[i];
    if (!t.param || !t.grad || !t.m || !t.v) return fail(GPT_ERR_INVALID, "tensor %d: a pointer is NULL", i);
    if (t.n <= 0) return fail(GPT_ERR_INVALID, "tensor %d: n must be positive", i);
    if (!aligned16(t.param) || !aligned16(t.grad) || !aligned16(t.m) || !aligned16(t.v) ||
        !aligned16(t.param_bf16))
      return fail(GPT_ERR_INVALID, "tensor %d: pointer not 16-byte aligned", i);
  }
  *out = reinterpret_cast<const OptTensor*>(tensors);
  return GPT_OK;
}

static int adamw_config(const gpt_adamw_config* cfg) {
  if (!cfg) return fail(GPT_ERR_INVALID, "cfg is NULL");
  const float hp[] = {cfg->lr, cfg->beta1, cfg->beta2, cfg->eps, cfg->weight_decay, cfg->max_norm};
  for (float x : hp)
    if (!std::isfinite(x)) return fail(GPT_ERR_INVALID, "non-finite hyperparameter");
  if (cfg->step < 1) return fail(GPT_ERR_INVALID, "step must be >= 1");
  if (!(cfg->beta1 >= 0.0f && cfg->beta1 < 1.0f && cfg->beta2 >= 0.0f && cfg->beta2 < 1.0f))
    return fail(GPT_ERR_INVALID, "betas must lie in [0, 1)");
  if (cfg->eps < 0.0f || cfg->lr < 0.0f || cfg->weight_decay < 0.0f)
    return fail(GPT_ERR_INVALID, "lr, eps and weight_decay must be non-negative");
  if (cfg->eps == 0.0f && cfg->beta2 == 0.0f) return fail(GPT_ERR_INVALID, "eps = 0 needs beta2 > 0");
  return GPT_OK;
}

size_t gpt_adamw_workspace_bytes(const gpt_adamw_tensor* tensors, int count) {
  const OptTensor* t = nullptr;
  if (adamw_tensors(tensors, count, &t)) return 0;
  return adamw_ws_bytes(t, count);
}

int gpt_adamw_step(const gpt_adamw_config* cfg, const gpt_adamw_tensor* tensors, int count, float* grad_norm,
                   void* ws, size_t ws_bytes, void* stream) {
  int st = adamw_config(cfg);
  if (st) return st;
  const OptTensor* t = nullptr;
  if ((st = adamw_tensors(tensors, count, &t))) return st;
  if (adamw_chunks(t, count) > (1L << 30)) return fail(GPT_ERR_UNSUPPORTED, "parameter set too large");
  const size_t need = adamw_ws_bytes(t, count);
  if (!ws || ws_bytes < need) return fail(GPT_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, need);
  if (!aligned16(ws) || !aligned16(grad_norm)) return fail(GPT_ERR_INVALID, "ws or grad_norm not 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  RUN("adamw", launch_adamw(t, count, cfg->lr, cfg->beta1, cfg->beta2, cfg->eps, cfg->weight_decay,
                            cfg->step, cfg->max_norm, grad_norm, ws, s));
  return GPT_OK;
}

int gpt_adamw_step_noalloc(const gpt_adamw_config* cfg, const gpt_adamw_tensor* tensors, int count,
                           float* grad_norm, void* stream) {
  int st = adamw_config(cfg);
  if (st) return st;
  const OptTensor* t = nullptr;
  if ((st = adamw_tensors(tensors, count, &t))) return st;
  const long chunks = adamw_chunks(t, count);
  if (chunks > ADAMW_NOALLOC_MAX_CHUNKS)
    return fail(GPT_ERR_UNSUPPORTED, "%ld chunks of 8192 elements exceed the %ld of the built-in scratch", chunks,
                ADAMW_NOALLOC_MAX_CHUNKS);
  if (!aligned16(grad_norm)) return fail(GPT_ERR_INVALID, "grad_norm not 16-byte aligned");
  void* scr = nullptr;
  HIPCHK(adamw_noalloc_scratch(&scr));
  hipStream_t s = static_cast<hipStream_t>(stream);
  // every partial and the clip factor the kernels read are written first by
  // this same call, so nothing in the scratch needs clearing
  RUN("adamw", launch_adamw(t, count, cfg->lr, cfg->beta1, cfg->beta2, cfg->eps, cfg->weight_decay,
                            cfg->step, cfg->max_norm, grad_norm, scr, s));
  return GPT_OK;
}

int gpt_embed_fwd(const gpt_config* cfg, int B, int T, const int32_t* ids, const void* wte, const void* wpe,
                  void* x0, void* stream) {
  Dims d;
  int st = check_bt(cfg, B, T, d);
  if (st) return st;
  if (!ids || !wte || !x0) return fail(GPT_ERR_INVALID, "ids, wte or x0 is NULL");
  if (!cfg->rope && !wpe) return fail(GPT_ERR_INVALID, "wpe is NULL with learned positions");
  hipStream_t s = static_cast<hipStream_t>(stream);
  RUN("embed_fwd", launch_embed_fwd(d.dtype, B, T, d.C, d.V, ids, wte, cfg->rope ? nullptr : wpe, x0, s));
  return GPT_OK;
}

int gpt_embed_bwd(const gpt_config* cfg, int B, int T, const int32_t* ids, const void* dx0, float* dwte, float* dwpe,
                  int accumulate, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_bt(cfg, B, T, d);
  if (st) return st;
  if (!ids || !dx0 || !dwte) return fail(GPT_ERR_INVALID, "ids, dx0 or dwte is NULL");
  const size_t need = embed_ws_bytes(d);
  if (!ws || ws_bytes < need) return fail(GPT_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  RUN("embed_bwd", launch_embed_bwd(d.dtype, B, T, d.C, d.V, cfg->block_size, ids, dx0, dwte, dwpe, accumulate, ws,
                                    ws_bytes, s));
  return GPT_OK;
}

int gpt_norm_fwd(const gpt_config* cfg, int N, const void* x, const void* w, const void* b, void* y, float* stats,
                 void* stream) {
  Dims d;
  int st = check_cfg(cfg, d);
  if (st) return st;
  if (N <= 0 || !x || !y) return fail(GPT_ERR_INVALID, "N <= 0 or x/y NULL");
  if (cfg->norm == GPT_NORM_LAYERNORM && !w) return fail(GPT_ERR_INVALID, "LayerNorm gain is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  RUN("normf_fwd", launch_norm_fwd(d.dtype, cfg->norm, N, d.C, x, w, opt(cfg, b), cfg->norm_eps, y, stats, s));
  return GPT_OK;
}

int gpt_norm_bwd(const gpt_config* cfg, int N, const void* x, const void* w, const void* dy, const void* resid,
                 void* dx, float* dw, float* db, int accumulate, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_cfg(cfg, d);
  if (st) return st;
  if (N <= 0 || !x || !dy || !dx) return fail(GPT_ERR_INVALID, "N <= 0 or x/dy/dx NULL");
  const bool ln = cfg->norm == GPT_NORM_LAYERNORM;
  if (ln && (!w || !dw)) return fail(GPT_ERR_INVALID, "LayerNorm gain or its gradient is NULL");
  d.N = N;
  const size_t need = norm_ws_bytes(d);
  if (ln && (!ws || ws_bytes < need)) return fail(GPT_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* colpart = static_cast<float*>(ws);
  const int nblk = norm_bwd_blocks(N);
  RUN("normf_bwd", launch_norm_bwd(d.dtype, cfg->norm, N, d.C, x, w, dy, resid, cfg->norm_eps, dx, colpart, ln, s));
  if (ln) {
    RUN("normf_cols", launch_colsum_finish(d.C, nblk, colpart, dw, accumulate, s));
    if (cfg->bias && db) RUN("normf_cols", launch_colsum_finish(d.C, nblk, colpart + (size_t)nblk * d.C, db, accumulate, s));
  }
  return GPT_OK;
}

}  // extern "C"
