// Host side of the C ABI declared in include/cacheblend.h: context, argument validation,
// the fetch/synchronize state machine, workspace planning and launch sequencing.
#include "../../include/cacheblend.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "cb_host.h"
#include "cb_kernels.h"

namespace {

thread_local std::string g_err;

cb_status vfail(cb_status st, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof buf, fmt, ap);
  g_err = buf;
  return st;
}

cb_status fail(cb_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}

cb_status hip_fail(hipError_t e, const char* what) {
  return fail(CB_EHIP, "%s: %s", what, hipGetErrorString(e));
}

enum LayerState { LS_IDLE = 0, LS_FETCHED = 1 };

struct ProfRec {
  int kernel;
  double work;
  hipEvent_t start, stop;
};

constexpr int kMaxProf = 16384;
constexpr int kGemmMaxSplits = 8;
constexpr int kAttnMaxSplits = 16;
constexpr int kAttnSmallRows = 64;     // kept sets this small (decode) get finer key splits:
constexpr int kAttnSmallSplits = 64;   // up to this many
constexpr int kPartialRows = 2048;  // split-K / split-KV partial buffers cover this many rows
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace

// Launch shape of the fetch kernel unless the caller sets one: 8 workgroups of 512 threads, two
// 16-byte pieces in flight per thread (512 KiB in flight).  Measured on MI355X, Qwen2.5-1.5B
// shape, blended prefills back to back (each prefetching while the previous one computes):
// 6.74 ms per prefill against 6.93 for 8 x 1024 x 4 and 7.25 for 32 x 64 x 1, although the last
// loads fastest alone (43 against 31 GB/s): the fetch slows the compute kernels while it runs,
// and spread over more CUs it slows them more.
constexpr cb::FetchLaunch kFetchLaunchDefault{8, 512, 2};
// CB_FETCH_AUTO takes the copy engine when the copies average this many bytes or more (one copy
// per run of chunks adjacent in host memory, per tensor K or V).
constexpr size_t kFetchCopyMinBytes = size_t(1) << 20;

struct cb_ctx {
  cb_model_desc d{};
  int device = 0;
  hipStream_t cs = nullptr, xs = nullptr;
  float2* rope = nullptr;  // [max_tokens][head_dim / 2]
  std::vector<cb_layer_weights> w;
  std::vector<char> have_w;
  // int8 layers: per-output-channel scales of w_qkv, w_o, w_gate_up, w_down (NULL: bf16 layer)
  struct Scales {
    const float *qkv, *o, *gate_up, *down;
  };
  std::vector<Scales> ws8;
  std::vector<hipEvent_t> fetch_ev;
  std::vector<hipEvent_t> release_ev;  // per layer: the compute stream is done with its fused K/V
  std::vector<int> state;
  int score_mode = CB_SCORE_L2;
  int fetch_mode = CB_FETCH_AUTO;
  cb::FetchLaunch fetch_launch = kFetchLaunchDefault;
  bool prof = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;

  int esize() const { return d.dtype == CB_BF16 ? 2 : 4; }
  bool bf16() const { return d.dtype == CB_BF16; }
};

namespace {

// Workspace layout (byte offsets), shared by blend_layer and layer_rest.
struct WsPlan {
  size_t x, fresh, dev, q, attn_o, attn_ml, didx, h1, mnorm, act, gpart, total;
  long attn_cap_rows;  // rows x splits the attention partials can hold
  long gpart_elems;    // fp32 elements of the split-K partial buffer
};

WsPlan plan_ws(const cb_model_desc& d, int n_tokens, int n_sel) {
  (void)n_tokens;
  WsPlan p{};
  const size_t es = d.dtype == CB_BF16 ? 2 : 4;
  const size_t ns = (size_t)std::max(n_sel, 1);
  const size_t qd = (size_t)d.n_q_heads * d.head_dim;
  const size_t kvd = (size_t)d.n_kv_heads * d.head_dim;
  const long prow = std::min<long>((long)ns, kPartialRows);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  p.x = take(ns * d.d_model * es);
  p.fresh = take(ns * (qd + 2 * kvd) * es);  // fresh K|V, or Q|K|V when every candidate is kept
  p.dev = take(ns * 4);
  p.q = take(ns * qd * es);
  // split-KV partials: up to kAttnMaxSplits key ranges per row, or kAttnSmallSplits for the
  // few rows of a decode step
  p.attn_cap_rows = std::max<long>(prow * kAttnMaxSplits, std::min<long>((long)ns, kAttnSmallRows) * kAttnSmallSplits);
  p.attn_o = take((size_t)p.attn_cap_rows * qd * 4);
  p.attn_ml = take((size_t)p.attn_cap_rows * d.n_q_heads * 2 * 4);
  p.didx = take(ns * 2 * 4);  // decode: kept positions and their local indices
  // layer_rest reuses the front of the workspace (blend_layer's buffers are dead by then)
  size_t blend_end = off;
  off = 0;
  p.h1 = take(ns * d.d_model * 4);
  p.mnorm = take(ns * d.d_model * es);
  p.act = take(ns * d.ffn_dim * es);
  off = std::max(off, blend_end);
  const size_t maxn = std::max<size_t>({(size_t)d.d_model, qd + 2 * kvd});
  p.gpart_elems = (long)(prow * maxn * kGemmMaxSplits);
  p.gpart = take((size_t)p.gpart_elems * 4);
  p.total = off;
  return p;
}

// Tile configuration and split-K factor of a bf16 GEMM (fp32 GEMMs never split).
void plan_gemm(cb::GemmArgs& g, bool bf, long cap_elems) {
  if (!bf) { g.splits = 1; return; }
  const cb::GemmPlan p = cb::gemm_plan(g.M, g.N, g.K, g.epi, cap_elems);
  g.cfg = p.cfg;
  g.splits = p.splits;
}

// Split-KV key ranges: 64 keys for the few rows of the decode kernel, 256 for up to 64 rows,
// 1024 below 1200 rows, 2048 below 2048 rows and 4800 from there on (measured best for the
// causal row-length mix of the fused prompt: at 2714 rows over 16,640 keys, 4 ranges of 4160
// keys against 5 of 3328 or 3 of 5568); fewer ranges when the partial buffer (2048 rows x 16
// ranges) cannot hold them all, so a dense prompt of 16,640 rows (layer 1) runs unsplit, its
// 520 row blocks x KV heads filling the chip by themselves.
void attn_splits(int n_q, int n_tok, int group, long cap_rows, int& splits, int& split_len) {
  const bool small = n_q <= kAttnSmallRows;
  const bool few = cb::attn_decode_fits(n_q, group);  // the decode kernel: 64-key ranges, any multiple of 16
  int len = few ? 64 : (small ? 256 : (n_q < 1200 ? 1024 : (n_q < 2048 ? 2048 : 4800)));
  int s = (n_tok + len - 1) / len;
  s = std::min(s, small ? kAttnSmallSplits : kAttnMaxSplits);
  while (s > 1 && (long)s * n_q > cap_rows) --s;
  const int gran = few ? 16 : 64;
  len = (n_tok + s - 1) / s;
  len = (len + gran - 1) / gran * gran;
  if (len <= 0) len = gran;
  splits = std::max(1, (n_tok + len - 1) / len);
  split_len = len;
}

struct Timed {
  cb_ctx* c;
  int kernel;
  double work;
  hipStream_t st;
  ProfRec* rec = nullptr;
  Timed(cb_ctx* c_, int k, double w, hipStream_t s = nullptr) : c(c_), kernel(k), work(w), st(s ? s : c_->cs) {
    if (!c->prof || c->ev_used + 2 > c->ev_pool.size()) return;
    c->recs.push_back(ProfRec{kernel, work, c->ev_pool[c->ev_used], c->ev_pool[c->ev_used + 1]});
    c->ev_used += 2;
    rec = &c->recs.back();
    // profiling is best effort: a failed record leaves this launch untimed (cb_profile_read
    // then reports the events' own error), it does not fail the launch it brackets
    (void)hipEventRecord(rec->start, st);
  }
  ~Timed() {
    if (rec) (void)hipEventRecord(rec->stop, st);
  }
};

// The compute stream is done with layer `layer`'s fused K/V (end of cb_blend_layer).
cb_status mark_release(cb_ctx* c, int layer) {
  if (c->xs == c->cs) return CB_OK;
  hipError_t e = hipEventRecord(c->release_ev[layer], c->cs);
  return e == hipSuccess ? CB_OK : hip_fail(e, "hipEventRecord(release)");
}

cb_status check_ctx(const cb_ctx* c) {
  if (!c) return fail(CB_EINVAL, "context is NULL");
  return CB_OK;
}

cb_status check_layer(const cb_ctx* c, int layer, bool need_w) {
  if (layer < 0 || layer >= c->d.n_layers)
    return fail(CB_EINVAL, "layer %d outside [0, %d)", layer, c->d.n_layers);
  if (need_w && !c->have_w[layer]) return fail(CB_ESTATE, "weights of layer %d not set", layer);
  return CB_OK;
}

cb_status check_offsets(const cb_ctx* c, const int32_t* offs, int n_chunks) {
  if (n_chunks < 0) return fail(CB_EINVAL, "n_chunks %d < 0", n_chunks);
  if (!offs) return fail(CB_EINVAL, "chunk_offsets_host is NULL");
  if (offs[0] != 0) return fail(CB_EINVAL, "chunk_offsets[0] = %d, must be 0", offs[0]);
  for (int i = 0; i < n_chunks; ++i)
    if (offs[i + 1] < offs[i]) return fail(CB_EINVAL, "chunk_offsets not monotone at %d", i);
  if (offs[n_chunks] > c->d.max_tokens) return fail(CB_ESHAPE, "context %d > max_tokens", offs[n_chunks]);
  return CB_OK;
}

}  // namespace

cb_status cbi_fail(cb_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}
hipStream_t cbi_compute_stream(const cb_ctx* c) { return c->cs; }
int cbi_device(const cb_ctx* c) { return c->device; }
const cb_model_desc* cbi_desc(const cb_ctx* c) { return &c->d; }

extern "C" {

const char* cb_last_error(void) { return g_err.c_str(); }

cb_status cb_create(const cb_model_desc* desc, int32_t device, void* compute_stream, void* copy_stream,
                    cb_ctx** out) {
  if (!desc || !out) return fail(CB_EINVAL, "desc or out is NULL");
  *out = nullptr;
  const cb_model_desc& d = *desc;
  if (d.n_layers <= 0 || d.d_model <= 0 || d.n_q_heads <= 0 || d.n_kv_heads <= 0 || d.head_dim <= 0 ||
      d.ffn_dim <= 0 || d.vocab_size <= 0 || d.max_tokens <= 0)
    return fail(CB_EINVAL, "model sizes must be positive");
  if (d.dtype != CB_F32 && d.dtype != CB_BF16) return fail(CB_EINVAL, "unknown dtype %d", d.dtype);
  if (d.n_q_heads % d.n_kv_heads) return fail(CB_ESHAPE, "n_q_heads not a multiple of n_kv_heads");
  if (d.head_dim != 64 && d.head_dim != 128) return fail(CB_EUNSUPPORTED, "head_dim %d (64 or 128)", d.head_dim);
  if (d.dtype == CB_BF16 && d.head_dim != 128) return fail(CB_EUNSUPPORTED, "bf16 path needs head_dim 128");
  const int G = d.n_q_heads / d.n_kv_heads;
  if (d.dtype == CB_BF16 && !(G == 1 || G == 2 || G == 4 || G == 6 || G == 7 || G == 8))
    return fail(CB_EUNSUPPORTED, "GQA group %d not instantiated", G);
  if (d.d_model % 128 || (d.n_q_heads * d.head_dim) % 128 || (2 * d.n_kv_heads * d.head_dim) % 128 ||
      d.ffn_dim % 64)
    return fail(CB_EUNSUPPORTED, "d_model, q width and 2*kv width must be multiples of 128, ffn of 64");
  if (!(d.rope_base > 0.f) || !(d.rms_eps >= 0.f)) return fail(CB_EINVAL, "rope_base / rms_eps invalid");

  hipError_t e = hipSetDevice(device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  cb_ctx* c = new cb_ctx();
  c->d = d;
  c->device = device;
  c->cs = (hipStream_t)compute_stream;
  c->xs = copy_stream ? (hipStream_t)copy_stream : c->cs;
  c->w.resize(d.n_layers);
  c->have_w.assign(d.n_layers, 0);
  c->ws8.assign(d.n_layers, cb_ctx::Scales{nullptr, nullptr, nullptr, nullptr});
  c->state.assign(d.n_layers, LS_IDLE);
  c->fetch_ev.assign(d.n_layers, nullptr);
  for (int l = 0; l < d.n_layers; ++l) {
    e = hipEventCreateWithFlags(&c->fetch_ev[l], hipEventDisableTiming);
    if (e != hipSuccess) { cb_destroy(c); return hip_fail(e, "hipEventCreate"); }
  }
  c->release_ev.assign(d.n_layers, nullptr);
  for (int l = 0; l < d.n_layers; ++l) {
    e = hipEventCreateWithFlags(&c->release_ev[l], hipEventDisableTiming);
    if (e != hipSuccess) { cb_destroy(c); return hip_fail(e, "hipEventCreate"); }
  }
  // RoPE table: angle p * base^(-2i/dh) and its cos/sin in double, stored as float.
  const int half = d.head_dim / 2;
  std::vector<float2> tab((size_t)d.max_tokens * half);
  for (int i = 0; i < half; ++i) {
    const double theta = std::pow((double)d.rope_base, -2.0 * i / d.head_dim);
    for (int p = 0; p < d.max_tokens; ++p) {
      const double ang = (double)p * theta;
      tab[(size_t)p * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
    }
  }
  e = hipMalloc((void**)&c->rope, tab.size() * sizeof(float2));
  if (e != hipSuccess) { cb_destroy(c); return hip_fail(e, "hipMalloc(rope table)"); }
  e = hipMemcpy(c->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice);
  if (e != hipSuccess) { cb_destroy(c); return hip_fail(e, "hipMemcpy(rope table)"); }
  *out = c;
  return CB_OK;
}

cb_status cb_destroy(cb_ctx* c) {
  if (!c) return CB_OK;
  // everything is released whatever fails; the first failure is reported (a stream that
  // cannot be synchronized, e.g. after a device fault, shows up here)
  hipError_t first = hipSuccess;
  auto note = [&](hipError_t e) {
    if (e != hipSuccess && first == hipSuccess) first = e;
  };
  note(hipSetDevice(c->device));
  if (c->cs) note(hipStreamSynchronize(c->cs));
  if (c->xs && c->xs != c->cs) note(hipStreamSynchronize(c->xs));
  if (!c->cs) note(hipDeviceSynchronize());
  for (hipEvent_t ev : c->fetch_ev)
    if (ev) note(hipEventDestroy(ev));
  for (hipEvent_t ev : c->ev_pool) note(hipEventDestroy(ev));
  for (hipEvent_t ev : c->release_ev)
    if (ev) note(hipEventDestroy(ev));
  if (c->rope) note(hipFree(c->rope));
  delete c;
  if (first != hipSuccess) return hip_fail(first, "cb_destroy (resources released)");
  return CB_OK;
}

cb_status cb_set_layer_weights(cb_ctx* c, int32_t layer, const cb_layer_weights* w) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if ((st = check_layer(c, layer, false))) return st;
  if (!w || !w->w_qkv || !w->w_o || !w->w_gate_up || !w->w_down || !w->g_attn || !w->g_ffn)
    return fail(CB_EINVAL, "a weight pointer of layer %d is NULL", layer);
  c->w[layer] = *w;
  c->have_w[layer] = 1;
  c->ws8[layer] = cb_ctx::Scales{nullptr, nullptr, nullptr, nullptr};
  return CB_OK;
}

cb_status cb_set_layer_weights_i8(cb_ctx* c, int32_t layer, const cb_layer_weights_i8* w) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if ((st = check_layer(c, layer, false))) return st;
  if (!c->bf16()) return fail(CB_EUNSUPPORTED, "int8 weights need a bf16 context");
  if (!w || !w->w_qkv || !w->w_o || !w->w_gate_up || !w->w_down || !w->s_qkv || !w->s_o || !w->s_gate_up ||
      !w->s_down || !w->g_attn || !w->g_ffn)
    return fail(CB_EINVAL, "a weight or scale pointer of layer %d is NULL", layer);
  const cb_model_desc& d = c->d;
  if (d.d_model % 16 || (d.n_q_heads * d.head_dim) % 16 || d.ffn_dim % 16)
    return fail(CB_EUNSUPPORTED, "int8 weight rows must be multiples of 16 bytes");
  c->w[layer] = cb_layer_weights{w->w_qkv, w->w_o, w->w_gate_up, w->w_down, w->g_attn, w->g_ffn};
  c->have_w[layer] = 1;
  c->ws8[layer] = cb_ctx::Scales{w->s_qkv, w->s_o, w->s_gate_up, w->s_down};
  return CB_OK;
}

cb_status cb_workspace_size(const cb_ctx* c, int32_t n_tokens, int32_t n_sel_max, size_t* bytes) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if (!bytes) return fail(CB_EINVAL, "bytes is NULL");
  if (n_tokens < 0 || n_sel_max < 0) return fail(CB_EINVAL, "negative size");
  if (n_sel_max > n_tokens) return fail(CB_ESHAPE, "n_sel_max %d > n_tokens %d", n_sel_max, n_tokens);
  *bytes = plan_ws(c->d, n_tokens, n_sel_max).total;
  return CB_OK;
}

cb_status cb_embed(cb_ctx* c, const int32_t* tokens, int32_t n, const void* table, float* hidden_out) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if (n < 0) return fail(CB_EINVAL, "n %d < 0", n);
  if (n == 0) return CB_OK;
  if (!tokens || !table || !hidden_out) return fail(CB_EINVAL, "NULL pointer");
  Timed t(c, CB_K_EMBED, (double)n * c->d.d_model * (c->esize() + 4));
  hipError_t e = cb::embed(tokens, n, table, c->d.vocab_size, c->d.d_model, c->bf16(), hidden_out, c->cs);
  return e == hipSuccess ? CB_OK : hip_fail(e, "embed launch");
}

}  // extern "C"

namespace {

// A fetch into layer l's fused buffers waits until the compute stream has finished the last
// cb_blend_layer of that layer enqueued before it (a no-op for a layer never blended), so a
// prefetch never overwrites rows that an earlier step still reads.
cb_status wait_release(cb_ctx* c, int layer) {
  if (c->xs == c->cs) return CB_OK;
  hipError_t e = hipStreamWaitEvent(c->xs, c->release_ev[layer], 0);
  return e == hipSuccess ? CB_OK : hip_fail(e, "hipStreamWaitEvent(release)");
}

cb_status check_fetch(cb_ctx* c, int layer, const int32_t* offs, int n_chunks, const int32_t* offs_dev,
                      const void* fused_k, const void* fused_v) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if ((st = check_layer(c, layer, false))) return st;
  if ((st = check_offsets(c, offs, n_chunks))) return st;
  if (c->state[layer] == LS_FETCHED) return fail(CB_ESTATE, "layer %d fetched twice without synchronize", layer);
  if (n_chunks > 0 && offs[n_chunks] > 0 && (!fused_k || !fused_v || !offs_dev)) return fail(CB_EINVAL, "NULL pointer");
  return CB_OK;
}

// Position update of the fetched rows on the copy stream, then the layer's event.
cb_status finish_fetch(cb_ctx* c, int layer, const void* src_k, const void* src_v, void* fused_k, void* fused_v,
                       const int32_t* offs_dev, int n_chunks, int n_ctx) {
  if (n_ctx > 0) {
    const bool inplace = src_k == fused_k;
    Timed t(c, CB_K_ROPE, (double)n_ctx * c->d.n_kv_heads * c->d.head_dim * c->esize() * (inplace ? 2.0 : 4.0), c->xs);
    hipError_t e = cb::rope_delta(src_k, src_v, fused_k, fused_v, n_ctx, c->d.n_kv_heads, c->d.head_dim, offs_dev,
                                  n_chunks, c->rope, c->d.max_tokens, c->bf16(), c->xs);
    if (e != hipSuccess) return hip_fail(e, "rope_delta launch");
  }
  hipError_t e = hipEventRecord(c->fetch_ev[layer], c->xs);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(fetch)");
  c->state[layer] = LS_FETCHED;
  return CB_OK;
}

}  // namespace

extern "C" {

namespace {

// Whether p lies in page-locked host memory that kernels may read at the same address (so a
// fetch kernel can read it over PCIe); anything else goes through the copy engine.
bool kernel_readable_host(const void* p) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // pageable memory is not an error here: clear it
    return false;
  }
  if (a.type != hipMemoryTypeHost || !a.devicePointer) return false;
  const char* host = a.hostPointer ? (const char*)a.hostPointer : (const char*)p;
  return (const char*)a.devicePointer + ((const char*)p - host) == (const char*)p;
}

}  // namespace

cb_status cb_set_fetch_mode(cb_ctx* c, int32_t mode) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if (mode != CB_FETCH_COPY && mode != CB_FETCH_KERNEL && mode != CB_FETCH_AUTO)
    return fail(CB_EINVAL, "unknown fetch mode %d", mode);
  c->fetch_mode = mode;
  return CB_OK;
}

cb_status cb_set_fetch_launch(cb_ctx* c, int32_t blocks, int32_t threads, int32_t unroll) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if (blocks == 0 && threads == 0 && unroll == 0) {
    c->fetch_launch = kFetchLaunchDefault;
    return CB_OK;
  }
  if (blocks < 1 || blocks > 1024 || threads < 64 || threads > 1024 || threads % 64 ||
      !(unroll == 1 || unroll == 2 || unroll == 4))
    return fail(CB_EINVAL, "fetch launch %d x %d threads, unroll %d: need 1..1024 workgroups of 64..1024 threads "
                "(a multiple of 64) and unroll 1, 2 or 4", blocks, threads, unroll);
  c->fetch_launch = cb::FetchLaunch{blocks, threads, unroll};
  return CB_OK;
}

cb_status cb_fetch_layer(cb_ctx* c, int32_t layer, const void* const* host_k, const void* const* host_v,
                         const int32_t* offs, int32_t n_chunks, const int32_t* offs_dev, void* fused_k,
                         void* fused_v) {
  cb_status st = check_fetch(c, layer, offs, n_chunks, offs_dev, fused_k, fused_v);
  if (st) return st;
  if (n_chunks > 0 && (!host_k || !host_v)) return fail(CB_EINVAL, "NULL pointer");
  const size_t row = (size_t)c->d.n_kv_heads * c->d.head_dim * c->esize();
  for (int ch = 0; ch < n_chunks; ++ch)
    if (offs[ch + 1] > offs[ch] && (!host_k[ch] || !host_v[ch])) return fail(CB_EINVAL, "chunk %d host pointer NULL", ch);
  // runs of chunks whose K rows, and whose V rows, follow one another in host memory: the
  // fused rows of consecutive chunks are adjacent too, so a run is one copy each for K and V
  std::vector<int> run_end;  // chunk index one past each run
  for (int ch = 0; ch < n_chunks; ++ch) {
    const size_t bytes = (size_t)(offs[ch + 1] - offs[ch]) * row;
    const bool joins = ch + 1 < n_chunks && (const char*)host_k[ch] + bytes == (const char*)host_k[ch + 1] &&
                       (const char*)host_v[ch] + bytes == (const char*)host_v[ch + 1];
    if (!joins) run_end.push_back(ch + 1);
  }
  bool direct = c->fetch_mode == CB_FETCH_KERNEL;
  if (c->fetch_mode == CB_FETCH_AUTO && n_chunks > 0)  // see cb_set_fetch_mode
    direct = (size_t)offs[n_chunks] * row / run_end.size() < kFetchCopyMinBytes;
  for (int ch = 0; direct && ch < n_chunks; ++ch)
    if (offs[ch + 1] > offs[ch] && !(kernel_readable_host(host_k[ch]) && kernel_readable_host(host_v[ch])))
      direct = false;
  if ((st = wait_release(c, layer))) return st;
  const int n_ctx = n_chunks > 0 ? offs[n_chunks] : 0;
  if (direct && n_ctx > 0) {  // one kernel per 64 chunks reads, rotates and writes the rows
    Timed t(c, CB_K_FETCH, (double)n_ctx * c->d.n_kv_heads * c->d.head_dim * c->esize() * 2.0, c->xs);
    for (int c0 = 0; c0 < n_chunks; c0 += cb::kFetchMaxChunks) {
      cb::FetchChunks F{};
      F.n = std::min(cb::kFetchMaxChunks, n_chunks - c0);
      for (int i = 0; i < F.n; ++i) {
        F.hk[i] = host_k[c0 + i];
        F.hv[i] = host_v[c0 + i];
        F.offs[i] = offs[c0 + i];
      }
      F.offs[F.n] = offs[c0 + F.n];
      hipError_t e = cb::fetch_rope(F, fused_k, fused_v, c->d.n_kv_heads, c->d.head_dim, c->rope, c->d.max_tokens,
                                    c->bf16(), c->fetch_launch, c->xs);
      if (e != hipSuccess) return hip_fail(e, "fetch kernel launch");
    }
    hipError_t e = hipEventRecord(c->fetch_ev[layer], c->xs);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(fetch)");
    c->state[layer] = LS_FETCHED;
    return CB_OK;
  }
  for (size_t r = 0, ch = 0; r < run_end.size(); ch = run_end[r++]) {
    const size_t bytes = (size_t)(offs[run_end[r]] - offs[ch]) * row;
    if (!bytes) continue;
    hipError_t e = hipMemcpyAsync((char*)fused_k + (size_t)offs[ch] * row, host_k[ch], bytes, hipMemcpyHostToDevice, c->xs);
    if (e == hipSuccess)
      e = hipMemcpyAsync((char*)fused_v + (size_t)offs[ch] * row, host_v[ch], bytes, hipMemcpyHostToDevice, c->xs);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(fetch)");
  }
  return finish_fetch(c, layer, fused_k, fused_v, fused_k, fused_v, offs_dev, n_chunks, n_chunks > 0 ? offs[n_chunks] : 0);
}

cb_status cb_fetch_layer_device(cb_ctx* c, int32_t layer, const void* cache_k, const void* cache_v,
                                const int32_t* offs, int32_t n_chunks, const int32_t* offs_dev, void* fused_k,
                                void* fused_v) {
  cb_status st = check_fetch(c, layer, offs, n_chunks, offs_dev, fused_k, fused_v);
  if (st) return st;
  const int n_ctx = n_chunks > 0 ? offs[n_chunks] : 0;
  if (n_ctx > 0 && (!cache_k || !cache_v)) return fail(CB_EINVAL, "NULL pointer");
  if ((cache_k == fused_k) != (cache_v == fused_v)) return fail(CB_EINVAL, "cache must alias fused for both K and V or for neither");
  if ((st = wait_release(c, layer))) return st;
  return finish_fetch(c, layer, cache_k, cache_v, fused_k, fused_v, offs_dev, n_chunks, n_ctx);
}

cb_status cb_rotate_layers(cb_ctx* c, int32_t first_layer, int32_t n_layers, const void* const* cache_k,
                           const void* const* cache_v, const int32_t* offs, int32_t n_chunks, const int32_t* offs_dev,
                           void* const* fused_k, void* const* fused_v) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if (n_layers < 0 || first_layer < 0 || first_layer + n_layers > c->d.n_layers)
    return fail(CB_EINVAL, "layers [%d, %d) outside [0, %d)", first_layer, first_layer + n_layers, c->d.n_layers);
  if ((st = check_offsets(c, offs, n_chunks))) return st;
  const int n_ctx = n_chunks > 0 ? offs[n_chunks] : 0;
  if (n_layers == 0 || n_ctx == 0) return CB_OK;
  if (!cache_k || !cache_v || !fused_k || !fused_v || !offs_dev) return fail(CB_EINVAL, "NULL pointer");
  const bool v_alias = cache_v[0] == fused_v[0];
  for (int i = 0; i < n_layers; ++i) {
    const int l = first_layer + i;
    if (c->state[l] == LS_FETCHED) return fail(CB_ESTATE, "layer %d has a pending fetch", l);
    if (!cache_k[i] || !cache_v[i] || !fused_k[i] || !fused_v[i]) return fail(CB_EINVAL, "NULL pointer (layer %d)", l);
    if ((cache_k[i] == fused_k[i]) != (cache_v[i] == fused_v[i]) || (cache_v[i] == fused_v[i]) != v_alias)
      return fail(CB_EINVAL, "cache must alias fused for both K and V or for neither, the same in every layer");
  }
  for (int b = 0; b < n_layers; b += cb::kRopeMaxLayers) {
    const int nb = std::min(cb::kRopeMaxLayers, n_layers - b);
    cb::RopeLayers L{};
    for (int i = 0; i < nb; ++i) {
      L.kc[i] = cache_k[b + i];
      L.vc[i] = cache_v[b + i];
      L.kf[i] = fused_k[b + i];
      L.vf[i] = fused_v[b + i];
    }
    Timed t(c, CB_K_ROPE, (double)nb * n_ctx * c->d.n_kv_heads * c->d.head_dim * c->esize() * (v_alias ? 2.0 : 4.0));
    hipError_t e = cb::rope_delta_layers(L, nb, n_ctx, c->d.n_kv_heads, c->d.head_dim, offs_dev, n_chunks, c->rope,
                                         c->d.max_tokens, v_alias ? 0 : 1, c->bf16(), c->cs);
    if (e != hipSuccess) return hip_fail(e, "rope_delta_layers launch");
  }
  return CB_OK;
}

cb_status cb_synchronize(cb_ctx* c, int32_t layer) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if ((st = check_layer(c, layer, false))) return st;
  if (c->state[layer] != LS_FETCHED) return CB_OK;
  if (c->xs != c->cs) {
    hipError_t e = hipStreamWaitEvent(c->cs, c->fetch_ev[layer], 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  c->state[layer] = LS_IDLE;
  return CB_OK;
}

cb_status cb_blend_layer(cb_ctx* c, int32_t layer, const float* hidden_sel, const void* x_sel, const void* kv_cached_k,
                         const void* kv_cached_v, void* kv_fused_k, void* kv_fused_v, const int32_t* offs_dev,
                         const int32_t* offs, int32_t n_chunks, const int32_t* sel_idx, int32_t n_sel,
                         int32_t n_query, float ratio, int32_t* new_sel_idx, int32_t* new_sel_local,
                         int32_t* n_new, void* out_sel, float* deviation, void* workspace, size_t ws_bytes) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if ((st = check_layer(c, layer, true))) return st;
  if ((st = check_offsets(c, offs, n_chunks))) return st;
  if (c->state[layer] == LS_FETCHED)
    return fail(CB_ESTATE, "layer %d has a pending fetch: call cb_synchronize first", layer);
  const cb_model_desc& d = c->d;
  const int n_ctx = offs[n_chunks];
  if (n_query < 0 || n_sel < 0) return fail(CB_EINVAL, "negative n_sel / n_query");
  const long n_tok = (long)n_ctx + n_query;
  if (n_tok > d.max_tokens) return fail(CB_ESHAPE, "prompt of %ld rows > max_tokens %d", n_tok, d.max_tokens);
  if (n_sel < n_query) return fail(CB_ESHAPE, "n_sel %d < n_query %d: every query row must be selected", n_sel, n_query);
  const int n_cand = n_sel - n_query;
  if (n_cand > n_ctx) return fail(CB_ESHAPE, "%d context rows selected > N_ctx %d", n_cand, n_ctx);
  if (!(ratio >= 0.f) || !std::isfinite(ratio)) return fail(CB_EINVAL, "ratio must be finite and >= 0");
  if (!n_new) return fail(CB_EINVAL, "n_new is NULL");
  if (n_sel > 0 && (!hidden_sel || !sel_idx || !new_sel_idx || !new_sel_local || !out_sel))
    return fail(CB_EINVAL, "NULL pointer");
  if (n_tok > 0 && (!kv_fused_k || !kv_fused_v)) return fail(CB_EINVAL, "kv_fused is NULL");
  if ((kv_cached_k == nullptr) != (kv_cached_v == nullptr)) return fail(CB_EINVAL, "kv_cached_k / _v: both or neither");
  if ((kv_cached_k == kv_fused_k) != (kv_cached_v == kv_fused_v))
    return fail(CB_EINVAL, "kv_cached must alias kv_fused for both K and V or for neither");
  if (n_chunks > 0 && kv_cached_k && !offs_dev) return fail(CB_EINVAL, "chunk_offsets_dev is NULL");
  const WsPlan wp = plan_ws(d, (int)n_tok, n_sel);
  if (!workspace || ws_bytes < wp.total)
    return fail(CB_ENOMEM, "workspace %zu bytes < %zu needed", ws_bytes, wp.total);

  long k = (long)std::floor((double)ratio * (double)n_ctx + 0.5);
  k = std::max(0L, std::min(k, (long)n_cand));
  const int nn = (int)k + n_query;
  *n_new = nn;
  if (n_sel == 0) return mark_release(c, layer);

  char* ws = (char*)workspace;
  const bool bf = c->bf16();
  const int es = c->esize();
  const int kvd = d.n_kv_heads * d.head_dim;
  const int qd = d.n_q_heads * d.head_dim;
  const int dm = d.d_model;
  const cb_layer_weights& W = c->w[layer];
  const cb_ctx::Scales& S8 = c->ws8[layer];
  hipError_t e;

  // 1. position update of the cached K (and copy of V) into the fused buffer
  if (n_ctx > 0 && kv_cached_k) {
    const bool inplace = kv_cached_k == kv_fused_k;
    Timed t(c, CB_K_ROPE, (double)n_ctx * kvd * es * (inplace ? 2.0 : 4.0));
    e = cb::rope_delta(kv_cached_k, kv_cached_v, kv_fused_k, kv_fused_v, n_ctx, d.n_kv_heads, d.head_dim, offs_dev,
                       n_chunks, c->rope, d.max_tokens, bf, c->cs);
    if (e != hipSuccess) return hip_fail(e, "rope_delta launch");
  }
  // 2. x = RMSNorm(hidden_sel), unless the caller passes it; a few rows (a decode step) go to the
  //    skinny products, which form x from hidden_sel as they load it (no launch of its own)
  const void* x = x_sel;
  const bool norm_on_load =
      !x && bf && cb::gemm_plan(n_sel, 2 * kvd, dm, cb::EPI_ROPE, 0).cfg == cb::GEMM_GEMV;
  auto set_a = [&](cb::GemmArgs& g) {
    if (norm_on_load) {
      g.A = nullptr; g.a_f32 = hidden_sel; g.a_gain = W.g_attn; g.a_eps = d.rms_eps;
    } else {
      g.A = x;
    }
  };
  if (!x && !norm_on_load) {
    void* xw = ws + wp.x;
    Timed t(c, CB_K_RMSNORM, (double)n_sel * dm * (4 + es));
    e = cb::rmsnorm(hidden_sel, dm, n_sel, dm, W.g_attn, d.rms_eps, xw, bf, c->cs);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
    x = xw;
  }
  // 3. fresh K | V of the selected rows (RoPE on K at the rows' positions).  When the layer keeps
  //    every candidate (k == n_cand: layer 1 and any layer whose ratio no longer narrows), the kept
  //    rows are exactly the selected rows, so Q is produced by the same GEMM (Q | K | V).
  const bool fuse_q = k == (long)n_cand;
  bool scattered = false;  // the fresh K/V already sit in the fused cache (see 3.)
  void* fresh = ws + wp.fresh;
  const int fresh_ld = fuse_q ? qd + 2 * kvd : 2 * kvd;
  void* fresh_kv = (char*)fresh + (fuse_q ? (size_t)qd * es : 0);
  {
    cb::GemmArgs g{};
    set_a(g); g.lda = dm; g.a_rows = nullptr;
    const size_t wes = S8.qkv ? 1 : es;  // bytes per weight
    g.B = fuse_q ? W.w_qkv : (const char*)W.w_qkv + (size_t)qd * dm * wes; g.ldb = dm;
    g.b_i8 = S8.qkv != nullptr; g.bscale = S8.qkv ? S8.qkv + (fuse_q ? 0 : qd) : nullptr;
    g.M = n_sel; g.N = fresh_ld; g.K = dm;
    g.partial = (float*)(ws + wp.gpart);
    g.epi = cb::EPI_ROPE; g.out = fresh; g.ldo = fresh_ld;
    plan_gemm(g, bf, wp.gpart_elems);
    g.pos = sel_idx; g.rope = c->rope; g.rope_cols = fuse_q ? qd + kvd : kvd; g.head_dim = d.head_dim;
    g.max_pos = d.max_tokens - 1;
    // every candidate kept and no deviation asked for: the deviation selects nothing, so the
    // product's epilogue writes the fresh K/V rows into the fused cache itself (and the kept set)
    if (fuse_q && bf && !deviation && kvd % 128 == 0 && qd % 128 == 0) {
      g.kv_k = kv_fused_k; g.kv_v = kv_fused_v; g.kv_col0 = qd; g.kvd = kvd; g.kv_rows = (int)n_tok;
      g.sel_out = new_sel_idx; g.local_out = new_sel_local;
      scattered = true;
    }
    Timed t(c, CB_K_GEMM_KV, 2.0 * g.M * g.N * g.K);
    e = bf ? cb::gemm_bf16(g, c->cs) : cb::gemm_f32(g, c->cs);
    if (e != hipSuccess) return hip_fail(e, "gemm(kv) launch");
  }
  // 4. deviation against the re-rotated cache, then scatter of the fresh rows; when every
  //    candidate is kept (fuse_q), the kept set is sel itself and the same kernel writes it
  // 5. gradual filtering otherwise: top-k of the context rows + every query row
  float* dev = deviation ? deviation : (float*)(ws + wp.dev);
  if (!scattered) {
    Timed t(c, CB_K_DEV_SCATTER, (double)n_sel * 2 * kvd * es * 2 + (double)n_cand * 2 * kvd * es);
    e = cb::dev_scatter(fresh_kv, fresh_ld, kv_fused_k, kv_fused_v, sel_idx, n_sel, n_cand, (int)n_tok, kvd,
                        n_ctx > 0 ? dev : nullptr, fuse_q ? new_sel_idx : nullptr, fuse_q ? new_sel_local : nullptr,
                        c->score_mode == CB_SCORE_COSINE, bf, c->cs);
    if (e != hipSuccess) return hip_fail(e, "dev_scatter launch");
  }
  if (!fuse_q) {
    Timed t(c, CB_K_TOPK, (double)n_cand * 4);
    e = cb::topk_select(dev, sel_idx, n_cand, n_query, (int)k, new_sel_idx, new_sel_local, c->cs);
    if (e != hipSuccess) return hip_fail(e, "topk launch");
  }
  if (nn == 0) return mark_release(c, layer);
  // 6a. Q of the kept rows (RoPE at their positions), unless the QKV GEMM already produced it
  void* q = fuse_q ? fresh : (void*)(ws + wp.q);
  const int q_ld = fuse_q ? fresh_ld : qd;
  if (!fuse_q) {
    cb::GemmArgs g{};
    set_a(g); g.lda = dm; g.a_rows = new_sel_local; g.a_rows_total = n_sel;
    g.B = W.w_qkv; g.ldb = dm;
    g.b_i8 = S8.qkv != nullptr; g.bscale = S8.qkv;
    g.M = nn; g.N = qd; g.K = dm;
    g.partial = (float*)(ws + wp.gpart);
    g.epi = cb::EPI_ROPE; g.out = q; g.ldo = qd;
    plan_gemm(g, bf, wp.gpart_elems);
    g.pos = new_sel_idx; g.rope = c->rope; g.rope_cols = qd; g.head_dim = d.head_dim; g.max_pos = d.max_tokens - 1;
    Timed t(c, CB_K_GEMM_Q, 2.0 * g.M * g.N * g.K);
    e = bf ? cb::gemm_bf16(g, c->cs) : cb::gemm_f32(g, c->cs);
    if (e != hipSuccess) return hip_fail(e, "gemm(q) launch");
  }
  // 6b. causal attention of the kept rows over the fused K/V
  {
    cb::AttnArgs a{};
    a.q = q; a.ldq = q_ld; a.qpos = new_sel_idx; a.n_q = nn;
    a.k = kv_fused_k; a.v = kv_fused_v; a.n_tok = (int)n_tok; a.hq = d.n_q_heads; a.hkv = d.n_kv_heads;
    a.dh = d.head_dim; a.out = out_sel; a.ldo = qd;
    a.part_o = (float*)(ws + wp.attn_o); a.part_ml = (float*)(ws + wp.attn_ml);
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d.head_dim));
    if (bf) attn_splits(nn, (int)n_tok, d.n_q_heads / d.n_kv_heads, wp.attn_cap_rows, a.splits, a.split_len);
    else { a.splits = 1; a.split_len = (int)std::max<long>(n_tok, 1); }
    // causal flops of the kept rows are not known on the host; the row count bounds them
    Timed t(c, CB_K_ATTN, 0.0);
    e = bf ? cb::attn_bf16(a, c->cs) : cb::attn_f32(a, c->cs);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
  }
  return mark_release(c, layer);
}

cb_status cb_decode_layer(cb_ctx* c, int32_t layer, const float* hidden_new, const void* x_new, void* kv_fused_k,
                          void* kv_fused_v, int32_t n_past, int32_t n_new, const int32_t* pos_dev, void* out_sel,
                          void* workspace, size_t ws_bytes) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if (n_past < 0 || n_new < 0) return fail(CB_EINVAL, "negative size");
  if ((long)n_past + n_new > c->d.max_tokens) return fail(CB_ESHAPE, "%d + %d rows > max_tokens", n_past, n_new);
  if (n_new > 0 && !pos_dev) return fail(CB_EINVAL, "pos_dev is NULL");
  const WsPlan wp = plan_ws(c->d, n_past + n_new, n_new);
  if (!workspace || ws_bytes < wp.total) return fail(CB_ENOMEM, "workspace %zu bytes < %zu needed", ws_bytes, wp.total);
  int32_t* idx = (int32_t*)((char*)workspace + wp.didx);
  const int32_t offs[2] = {0, n_past};
  int32_t nn = 0;
  // every past row is already-fused context (nothing to re-rotate, nothing to rank); the new
  // rows are the query rows and are all kept
  return cb_blend_layer(c, layer, hidden_new, x_new, nullptr, nullptr, kv_fused_k, kv_fused_v, nullptr, offs,
                        n_past > 0 ? 1 : 0, pos_dev, n_new, n_new, 0.f, idx, idx + std::max(n_new, 1), &nn, out_sel,
                        nullptr, workspace, ws_bytes);
}

cb_status cb_workspace_views(const cb_ctx* c, int32_t n_sel, int32_t all_kept, cb_ws_views* out) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if (n_sel < 0 || !out) return fail(CB_EINVAL, "negative n_sel or NULL output");
  const WsPlan wp = plan_ws(c->d, n_sel, n_sel);
  const int qd = c->d.n_q_heads * c->d.head_dim, kvd = c->d.n_kv_heads * c->d.head_dim;
  out->q_offset = all_kept ? wp.fresh : wp.q;  // see steps 3 and 6a of cb_blend_layer
  out->q_ld = all_kept ? qd + 2 * kvd : qd;
  out->h1_offset = wp.h1;
  out->act_offset = wp.act;
  return CB_OK;
}

cb_status cb_layer_rest(cb_ctx* c, int32_t layer, const float* hidden_sel, int32_t n_sel,
                        const int32_t* new_sel_local, int32_t n_new, const void* out_sel, float* hidden_next,
                        void* x_next, void* workspace, size_t ws_bytes) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if ((st = check_layer(c, layer, true))) return st;
  const cb_model_desc& d = c->d;
  if (n_sel < 0 || n_new < 0) return fail(CB_EINVAL, "negative size");
  if (n_new > n_sel) return fail(CB_ESHAPE, "n_new %d > n_sel %d", n_new, n_sel);
  if (n_new == 0) return CB_OK;
  if (!hidden_sel || !new_sel_local || !out_sel || !hidden_next) return fail(CB_EINVAL, "NULL pointer");
  if ((const void*)hidden_next == (const void*)hidden_sel) return fail(CB_EINVAL, "hidden_next aliases hidden_sel");
  if (x_next && (layer + 1 >= d.n_layers || !c->have_w[layer + 1]))
    return fail(CB_ESTATE, "x_next needs the weights of layer %d", layer + 1);
  const WsPlan wp = plan_ws(d, n_sel, n_sel);
  if (!workspace || ws_bytes < wp.total) return fail(CB_ENOMEM, "workspace %zu bytes < %zu needed", ws_bytes, wp.total);
  char* ws = (char*)workspace;
  const bool bf = c->bf16();
  const int es = c->esize();
  const int dm = d.d_model, qd = d.n_q_heads * d.head_dim, ff = d.ffn_dim;
  const cb_layer_weights& W = c->w[layer];
  const cb_ctx::Scales& S8 = c->ws8[layer];
  float* h1 = (float*)(ws + wp.h1);
  void* mn = ws + wp.mnorm;
  void* act = ws + wp.act;
  // a few rows (a decode step): the skinny gate/up product forms RMSNorm(h1) as it loads h1
  const bool norm_on_load = bf && cb::gemm_plan(n_new, 2 * ff, dm, cb::EPI_SWIGLU, 0).cfg == cb::GEMM_GEMV;
  hipError_t e;
  {  // h1 = hidden_sel[new_sel_local] + out_sel W_o^T, and mn = RMSNorm(h1) (fused for bf16)
    cb::GemmArgs g{};
    g.A = out_sel; g.lda = qd; g.B = W.w_o; g.ldb = qd;
    g.b_i8 = S8.o != nullptr; g.bscale = S8.o;
    g.M = n_new; g.N = dm; g.K = qd;
    g.partial = (float*)(ws + wp.gpart);
    g.epi = cb::EPI_RESID; g.out = h1; g.ldo = dm; g.resid = hidden_sel; g.ldr = dm; g.resid_rows = new_sel_local;
    plan_gemm(g, bf, wp.gpart_elems);
    if (bf && !norm_on_load) { g.norm_g = W.g_ffn; g.norm_eps = d.rms_eps; g.norm_out = mn; }
    Timed t(c, CB_K_GEMM_O, 2.0 * g.M * g.N * g.K);
    e = bf ? cb::gemm_bf16(g, c->cs) : cb::gemm_f32(g, c->cs);
    if (e != hipSuccess) return hip_fail(e, "gemm(o) launch");
  }
  if (!bf) {
    Timed t(c, CB_K_RMSNORM, (double)n_new * dm * (4 + es));
    e = cb::rmsnorm(h1, dm, n_new, dm, W.g_ffn, d.rms_eps, mn, bf, c->cs);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
  }
  {  // act = silu(m W_gate^T) * (m W_up^T)
    cb::GemmArgs g{};
    g.A = mn; g.lda = dm; g.B = W.w_gate_up; g.ldb = dm; g.swiglu_ffn = ff;
    if (norm_on_load) { g.A = nullptr; g.a_f32 = h1; g.a_gain = W.g_ffn; g.a_eps = d.rms_eps; }
    g.b_i8 = S8.gate_up != nullptr; g.bscale = S8.gate_up;
    g.M = n_new; g.N = 2 * ff; g.K = dm;
    g.epi = cb::EPI_SWIGLU; g.out = act; g.ldo = ff;
    plan_gemm(g, bf, 0);
    Timed t(c, CB_K_GEMM_GATE_UP, 2.0 * g.M * g.N * g.K);
    e = bf ? cb::gemm_bf16(g, c->cs) : cb::gemm_f32(g, c->cs);
    if (e != hipSuccess) return hip_fail(e, "gemm(gate_up) launch");
  }
  {  // hidden_next = h1 + act W_down^T
    cb::GemmArgs g{};
    g.A = act; g.lda = ff; g.B = W.w_down; g.ldb = ff;
    g.b_i8 = S8.down != nullptr; g.bscale = S8.down;
    g.M = n_new; g.N = dm; g.K = ff;
    g.partial = (float*)(ws + wp.gpart);
    g.epi = cb::EPI_RESID; g.out = hidden_next; g.ldo = dm; g.resid = h1; g.ldr = dm;
    plan_gemm(g, bf, wp.gpart_elems);
    if (bf && x_next) { g.norm_g = c->w[layer + 1].g_attn; g.norm_eps = d.rms_eps; g.norm_out = x_next; }
    Timed t(c, CB_K_GEMM_DOWN, 2.0 * g.M * g.N * g.K);
    e = bf ? cb::gemm_bf16(g, c->cs) : cb::gemm_f32(g, c->cs);
    if (e != hipSuccess) return hip_fail(e, "gemm(down) launch");
  }
  if (!bf && x_next) {
    Timed t(c, CB_K_RMSNORM, (double)n_new * dm * (4 + es));
    e = cb::rmsnorm(hidden_next, dm, n_new, dm, c->w[layer + 1].g_attn, d.rms_eps, x_next, bf, c->cs);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
  }
  return CB_OK;
}

cb_status cb_set_score_mode(cb_ctx* c, int32_t mode) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if (mode != CB_SCORE_L2 && mode != CB_SCORE_COSINE) return fail(CB_EINVAL, "unknown score mode %d", mode);
  c->score_mode = mode;
  return CB_OK;
}

cb_status cb_seam_select(const int32_t* offs, int32_t n_chunks, int32_t n_query, int32_t window, int32_t* out,
                         int32_t capacity, int32_t* n_out) {
  if (!offs || !n_out || (capacity > 0 && !out)) return fail(CB_EINVAL, "NULL pointer");
  if (n_chunks < 0 || n_query < 0 || window < 0 || capacity < 0) return fail(CB_EINVAL, "negative size");
  if (offs[0] != 0) return fail(CB_EINVAL, "chunk_offsets[0] = %d, must be 0", offs[0]);
  for (int c = 0; c < n_chunks; ++c)
    if (offs[c + 1] < offs[c]) return fail(CB_EINVAL, "chunk_offsets not monotone at %d", c);
  long n = 0;
  for (int c = 0; c < n_chunks; ++c) n += std::min<long>(window, offs[c + 1] - offs[c]);
  n += n_query;
  *n_out = (int32_t)n;
  if (n > capacity) return fail(CB_ESHAPE, "%ld seam rows > capacity %d", n, capacity);
  int32_t* o = out;
  for (int c = 0; c < n_chunks; ++c)
    for (int32_t p = std::max(offs[c], offs[c + 1] - window); p < offs[c + 1]; ++p) *o++ = p;
  for (int32_t q = 0; q < n_query; ++q) *o++ = offs[n_chunks] + q;
  return CB_OK;
}

cb_status cb_plan_ratio(int32_t n_ctx, int32_t n_layers, double kvb, double bw, double pre, double lat, float r_min,
                        float r_max, cb_ratio_plan* out) {
  if (!out) return fail(CB_EINVAL, "out is NULL");
  if (n_ctx <= 0 || n_layers <= 0 || !(kvb > 0) || !(bw > 0) || !(pre > 0) || !(lat >= 0))
    return fail(CB_EINVAL, "sizes, bandwidth and prefill time must be positive, latency >= 0");
  if (!(r_min >= 0.f) || !(r_max >= r_min) || !(r_max <= 1.f)) return fail(CB_EINVAL, "need 0 <= r_min <= r_max <= 1");
  const double t_pre_layer = (double)n_ctx * pre / n_layers;
  const double be = kvb * n_layers / pre;
  cb_ratio_plan p{};
  p.break_even_bandwidth = be;
  if (bw <= be) {
    p.load = 0;
    p.ratio = 1.f;
    p.t_load_layer = 0.0;
    p.t_recompute_layer = p.t_layer = t_pre_layer;
  } else {
    p.load = 1;
    p.t_load_layer = (double)n_ctx * kvb / bw + lat;
    const double r = std::min<double>(std::max<double>(p.t_load_layer / t_pre_layer, r_min), r_max);
    p.ratio = (float)r;
    p.t_recompute_layer = r * t_pre_layer;
    p.t_layer = std::max(p.t_load_layer, p.t_recompute_layer);
  }
  p.t_total = n_layers * p.t_layer;
  *out = p;
  return CB_OK;
}

cb_status cb_plan_ratio_measured(int32_t n_layers, double kv_bytes_layer, double bw, double lat, double t_first,
                                 double t_select, double t_full, double t_fixed, double contention, float r_min,
                                 float r_max, cb_ratio_plan* out) {
  if (!out) return fail(CB_EINVAL, "out is NULL");
  if (n_layers <= 0 || !(kv_bytes_layer > 0) || !(bw > 0) || !(lat >= 0) || !(t_first >= 0) || !(t_select >= 0) ||
      !(t_full > 0) || !(t_fixed >= 0) || !(t_fixed <= t_full) || !(contention >= 0))
    return fail(CB_EINVAL, "need n_layers, bytes, bandwidth, t_full > 0, latency, t_first, t_select, contention >= 0, "
                           "0 <= t_fixed <= t_full");
  if (!(r_min >= 0.f) || !(r_max >= r_min) || !(r_max <= 1.f)) return fail(CB_EINVAL, "need 0 <= r_min <= r_max <= 1");
  const double slope = t_full - t_fixed;
  const double tl = kv_bytes_layer / bw + lat;
  auto layer = [&](double tr) { return std::max(tl, tr) + contention * std::min(tl, tr); };
  cb_ratio_plan p{};
  p.break_even_bandwidth = kv_bytes_layer / t_full;
  if (layer(t_fixed + (double)r_min * slope) >= t_full) {  // loading cannot beat recomputing the layer
    p.load = 0;
    p.ratio = 1.f;
    p.t_recompute_layer = p.t_layer = t_full;
    p.t_total = t_first + (double)(n_layers - 1) * p.t_layer;
  } else {
    p.load = 1;
    p.t_load_layer = tl;
    const double r = std::min<double>(std::max<double>((tl - t_fixed) / slope, r_min), r_max);
    p.ratio = (float)r;
    p.t_recompute_layer = t_fixed + r * slope;
    p.t_layer = layer(p.t_recompute_layer);
    p.t_total = t_first + t_select + (double)(n_layers - 1) * p.t_layer;
  }
  *out = p;
  return CB_OK;
}

cb_status cb_profile_enable(cb_ctx* c, int32_t on) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if (on) {
    if (c->ev_pool.empty()) {
      c->ev_pool.resize(2 * kMaxProf);
      for (auto& ev : c->ev_pool) {
        hipError_t e = hipEventCreate(&ev);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate(profile)");
      }
    }
    c->recs.clear();
    c->recs.reserve(kMaxProf);
    c->ev_used = 0;
  }
  c->prof = on != 0;
  return CB_OK;
}

cb_status cb_profile_read(cb_ctx* c, int32_t kernel_id, double* total_ms, int64_t* launches, double* work) {
  cb_status st = check_ctx(c);
  if (st) return st;
  if (kernel_id < 0 || kernel_id >= CB_K_COUNT) return fail(CB_EINVAL, "kernel id %d", kernel_id);
  double ms = 0, wk = 0;
  int64_t n = 0;
  for (const ProfRec& r : c->recs) {
    if (r.kernel != kernel_id) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(profile)");
    float t = 0;
    e = hipEventElapsedTime(&t, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    ms += t;
    wk += r.work;
    ++n;
  }
  if (total_ms) *total_ms = ms;
  if (launches) *launches = n;
  if (work) *work = wk;
  return CB_OK;
}

}  // extern "C"
