// C ABI: argument checks, buffer carving and the streaming state machine.
// The schedule is host arithmetic only (lengths never depend on device data:
// compression always leaves exactly spkcache_len frames), so every call just
// enqueues kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>

#include "kernels.h"
#include "model.h"

using namespace sf;
using namespace sfm;

namespace {

inline hipStream_t HS(void* s) { return static_cast<hipStream_t>(s); }
inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
inline sf_status launched() {
  if (take_gemm_failure()) return SF_ENOMEM;
  return hipGetLastError() == hipSuccess ? SF_OK : SF_EHIP;
}

bool valid_stream_config(const sf_stream_config* c) {
  if (!c) return false;
  if (c->chunk_len < 1 || c->right_context < 0 || c->fifo_len < 0 || c->update_period < 1 ||
      c->spkcache_len < 1 || c->n_sil_per_spk < 0)
    return false;
  return true;
}

int stream_cap(const sf_stream_config* c) {
  return c->spkcache_len + c->fifo_len + c->chunk_len + c->right_context;
}

long long ring_cap_for(const sf_stream_config* c) {
  long long need = 1280LL * (c->chunk_len + c->right_context) + 2048, cap = 1;
  while (cap < need) cap <<= 1;
  return cap;
}

// Byte layout of the state buffer.
struct StateLayout {
  size_t e, p, ph, sum, cnt, slots, ring, total;
};
StateLayout state_layout(const sf_model* m, const sf_stream_config* c, int B) {
  const size_t cap = stream_cap(c), S = m->cfg.n_spk, D = 512;
  StateLayout L{};
  L.e = al256((size_t)B * cap * D * 4);
  L.p = al256((size_t)B * cap * S * 4);
  L.ph = al256((size_t)B * cap * 4);
  L.sum = al256((size_t)B * D * 8);
  L.cnt = al256((size_t)B * 4);
  L.slots = al256((size_t)B * cap * 4);
  L.ring = al256((size_t)B * ring_cap_for(c) * 4);
  L.total = 2 * (L.e + L.p + L.ph) + L.sum + L.cnt + L.slots + L.ring;
  return L;
}

void bind_state(sf_stream* st, char* base) {
  const StateLayout L = state_layout(st->m, &st->sc, st->B);
  char* p = base;
  for (int i = 0; i < 2; ++i) {
    st->E[i] = reinterpret_cast<float*>(p); p += L.e;
    st->P[i] = reinterpret_cast<float*>(p); p += L.p;
    st->ph[i] = reinterpret_cast<int*>(p); p += L.ph;
  }
  st->sil_sum = reinterpret_cast<double*>(p); p += L.sum;
  st->sil_cnt = reinterpret_cast<int*>(p); p += L.cnt;
  st->slots = reinterpret_cast<int*>(p); p += L.slots;
  st->ring = reinterpret_cast<float*>(p);
}

void reset_host(sf_stream* st) {
  st->cur = 0;
  st->Lc = st->Lf = st->Lp = 0;
  st->steps = st->emitted = st->recv = st->pending = 0;
  st->enc_done = 0;
  st->finished = false;
  st->rows_only = false;
}

// Lengths after the cache update of a step that scored n_chunk look-ahead
// rows: FIFO append, the pop rule n = min(len, max(update_period, len -
// fifo_len)) ("Streaming Sortformer Diarizer" model card, Streaming
// Architecture and Configurations), and compression back to spkcache_len.
struct Lens {
  int Lc, Lf, Lp, popped;
  bool compress;
};
Lens lens_after_update(const sf_stream_config& c, int Lc, int Lf, int Lp, int n_chunk) {
  Lens r{Lc, Lf + n_chunk, Lp - n_chunk, 0, false};
  if (r.Lf > c.fifo_len) {
    r.popped = std::min(r.Lf, std::max(c.update_period, r.Lf - c.fifo_len));
    r.Lc += r.popped;
    r.Lf -= r.popped;
  }
  if (r.Lc > c.spkcache_len) {
    r.compress = true;
    r.Lc = c.spkcache_len;
  }
  return r;
}

void reset_device(sf_stream* st, hipStream_t s) {
  const long long rows = (long long)st->B * st->cap;
  fill_i32(st->ph[0], rows, 0, s);
  fill_i32(st->ph[1], rows, 0, s);
  fill_f64(st->sil_sum, (long long)st->B * st->D, 0.0, s);
  fill_i32(st->sil_cnt, st->B, 0, s);
}

// FIFO refresh/append, pop with silence statistics, compression.
void state_update(sf_stream* st, const float* probs, int W, int n_chunk, hipStream_t s) {
  const int S = st->S, D = st->D, B = st->B, cap = st->cap, cur = st->cur;
  const Lens n = lens_after_update(st->sc, st->Lc, st->Lf, st->Lp, n_chunk);
  refresh_probs(probs, W, S, B, st->Lc, st->Lf + n_chunk, st->P[cur], st->ph[cur], cap, s);
  if (n.popped > 0)
    silence_update(st->E[cur], st->P[cur], cap, D, S, B, st->Lc, n.popped, st->sil_sum,
                   st->sil_cnt, s);
  if (n.compress) {
    const int C = st->sc.spkcache_len, per = C / S;
    const int k = std::max(0, per - st->sc.n_sil_per_spk);
    compress_cache(st->E[cur], st->P[cur], st->ph[cur], cap, D, S, B, st->Lc + n.popped,
                   n.Lf + n.Lp, st->sil_sum, st->sil_cnt, C, per, k, st->E[cur ^ 1],
                   st->P[cur ^ 1], st->ph[cur ^ 1], st->slots, s);
    st->cur ^= 1;
  }
  st->Lc = n.Lc;
  st->Lf = n.Lf;
  st->Lp = n.Lp;
}

// Releases the cached graphs. A replay may still be queued on any stream the
// caller used, so the device is drained first (only when graphs exist: the
// workspace changed, graphs were switched off, or the state is destroyed).
void drop_graphs(sf_stream* st) {
  if (st->graphs.empty()) return;
  (void)hipDeviceSynchronize();
  for (auto& kv : st->graphs) (void)hipGraphExecDestroy(static_cast<hipGraphExec_t>(kv.second));
  st->graphs.clear();
}

// Rows per stream of the window forward: the window itself, or the whole
// capacity when windows are padded to one fixed size.
int window_rows(const sf_stream* st) {
  return st->fixed_window ? st->cap : st->Lc + st->Lf + st->Lp;
}

// Window copy + encoder for the current state, enqueued on s. A fixed window
// copies all cap rows, zeroing those at or past the valid length that the
// kernels read from enc.nv (set by the caller of this function).
void window_forward(sf_stream* st, EncWs& enc, hipStream_t s) {
  const int W = st->Lc + st->Lf + st->Lp;
  if (st->fixed_window) {
    copy_rows_nv(st->E[st->cur], (long long)st->cap * st->D, st->D, enc.x,
                 (long long)st->cap * st->D, st->D, st->B, st->cap, st->D, enc.nv, s);
    encode(st->m, enc, st->B, st->cap, st->cap, s, false, enc.nv);
    return;
  }
  copy_rows(st->E[st->cur], (long long)st->cap * st->D, st->D, enc.x, (long long)W * st->D, st->D,
            st->B, W, st->D, s);
  encode(st->m, enc, st->B, W, W, s);
}

// Runs window_forward, through a cached graph when enabled. Returns false if
// capture or instantiation failed (then the direct launch path was used).
bool window_forward_graph(sf_stream* st, EncWs& enc, const void* ws, hipStream_t s) {
  const int W = window_rows(st);
  if (ws != st->graph_ws) {  // graphs of one workspace at a time: at most 2 per window size
    drop_graphs(st);
    st->graph_ws = ws;
  }
  const auto key = std::make_tuple(W, st->cur, ws);
  auto it = st->graphs.find(key);
  if (it == st->graphs.end()) {
    if (!st->cap_stream) {
      hipStream_t cs = nullptr;
      if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return false;
      st->cap_stream = cs;
    }
    hipStream_t cs = static_cast<hipStream_t>(st->cap_stream);
    hipGraph_t g = nullptr;
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) return false;
    window_forward(st, enc, cs);
    if (hipStreamEndCapture(cs, &g) != hipSuccess || !g) return false;
    hipGraphExec_t ex = nullptr;
    const bool ok = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0) == hipSuccess;
    (void)hipGraphDestroy(g);
    if (!ok) return false;
    it = st->graphs.emplace(key, ex).first;
  }
  return hipGraphLaunch(static_cast<hipGraphExec_t>(it->second), s) == hipSuccess;
}

// One window forward on the current state, emitting the chunk rows.
void step_core(sf_stream* st, int n_chunk, float* out, long long out_bstride, EncWs& enc,
               const void* ws, hipStream_t s) {
  const sf_model* m = st->m;
  const int S = st->S, B = st->B;
  const int W = window_rows(st);  // row pitch of the window's outputs
  if (st->fixed_window) fill_i32(enc.nv, 1, st->Lc + st->Lf + st->Lp, s);
  bool done = false;
  if (st->use_graphs && ws && !profiling()) done = window_forward_graph(st, enc, ws, s);
  if (!done) {
    (void)hipGetLastError();  // a failed capture must not leak its status
    window_forward(st, enc, s);
  }
  const int r0 = st->Lc + st->Lf;
  if (m->cfg.arch == SF_ARCH_SORTFORMER)
    copy_rows(enc.probs + (size_t)r0 * S, (long long)W * S, S, out, out_bstride, S, B, n_chunk, S, s);
  else if (m->out_stride == 1)
    copy_rows(enc.probs10 + (size_t)8 * r0 * S, (long long)8 * W * S, S, out, out_bstride, S, B,
              8 * n_chunk, S, s);
  else
    pool_rows(enc.probs10 + (size_t)8 * r0 * S, (long long)8 * W * S, out, out_bstride, B,
              8 * n_chunk / m->out_stride, m->out_stride, S, s);
  state_update(st, enc.probs, W, n_chunk, s);
}

size_t stream_ws_bytes(const sf_model* m, const sf_stream_config* c, int B) {
  return al256(enc_ws_bytes(m, B, stream_cap(c))) +
         al256(pre_ws_bytes(m, B, c->chunk_len + c->right_context));
}

int frames_of(long long n_samples) {
  const long long T = n_samples / 160;
  return (int)((T + 7) / 8);
}

}  // namespace

extern "C" {

const char* sortformer_status_string(sf_status s) {
  switch (s) {
    case SF_OK: return "ok";
    case SF_EINVAL: return "invalid argument";
    case SF_ESHAPE: return "size outside the supported range";
    case SF_ENOMEM: return "caller buffer too small";
    case SF_EHIP: return "HIP runtime error";
    case SF_ESTATE: return "call not allowed in the current stream state";
    case SF_EUNSUPPORTED: return "unsupported combination";
    default: return "unknown status";
  }
}

sf_status sortformer_stream_preset(const char* name, sf_stream_config* out) {
  if (!name || !out) return SF_EINVAL;
  struct P { const char* n; int v[5]; };
  static const P presets[] = {{"very_high", {340, 40, 40, 300, 188}},
                              {"high", {124, 1, 124, 124, 188}},
                              {"low", {6, 7, 188, 144, 188}},
                              {"ultra_low", {3, 1, 188, 144, 188}},
                              {"very_low", {6, 2, 188, 144, 188}},
                              {"nemotron_offline", {380, 0, 188, 192, 188}}};
  for (const P& p : presets)
    if (std::strcmp(p.n, name) == 0) {
      *out = sf_stream_config{p.v[0], p.v[1], p.v[2], p.v[3], p.v[4], 3};
      return SF_OK;
    }
  return SF_EINVAL;
}

size_t sortformer_weight_bytes(const sf_model_config* cfg) { return weight_bytes(cfg); }

sf_status sortformer_init(const sf_model_config* cfg, uint64_t seed, void* d_weights,
                          size_t bytes, void* stream, sf_model** out) {
  if (!valid_config(cfg) || !d_weights || !out) return SF_EINVAL;
  if (reinterpret_cast<uintptr_t>(d_weights) % 256) return SF_EINVAL;
  if (bytes < weight_bytes(cfg)) return SF_ENOMEM;
  sf_model* m = new (std::nothrow) sf_model{};
  if (!m) return SF_ENOMEM;
  m->cfg = *cfg;
  m->seed = seed;
  m->out_stride = 1;
  const sf_status st = init_model(m, d_weights, bytes, HS(stream));
  if (st != SF_OK) {
    delete m;
    return st;
  }
  *out = m;
  return SF_OK;
}

void sortformer_free(sf_model* m) { delete m; }

sf_status sortformer_get_config(const sf_model* m, sf_model_config* out) {
  if (!m || !out) return SF_EINVAL;
  *out = m->cfg;
  return SF_OK;
}

sf_status sortformer_get_metadata(const sf_model* m, sf_model_metadata* out) {
  if (!m || !out) return SF_EINVAL;
  const bool sfm_ = m->cfg.arch == SF_ARCH_SORTFORMER;
  sf_model_metadata d{};
  d.window_stride = 0.01;
  d.output_frame_s = sfm_ ? 0.08 : 0.01;
  d.sample_rate = 16000;
  d.subsampling_factor = 8;
  d.fc_d_model = sfm_ ? 512 : 0;
  d.tf_d_model = sfm_ ? 192 : 512;
  d.max_num_of_spks = m->cfg.n_spk;
  d.spkcache_len = 188;
  d.n_mels = 128;
  d.n_fft = 512;
  d.win_length = 400;
  d.hop_length = 160;
  d.n_conformer_layers = sfm_ ? 17 : 0;
  d.n_transformer_layers = sfm_ ? 18 : 31;
  d.n_heads = 8;
  d.max_window = SF_MAX_WINDOW;
  *out = d;
  return SF_OK;
}

int32_t sortformer_num_tensors(const sf_model* m) { return m ? (int32_t)m->list.size() : 0; }

sf_status sortformer_tensor_info(const sf_model* m, int32_t i, char* name, int32_t cap,
                                 int64_t* numel) {
  if (!m || i < 0 || i >= (int32_t)m->list.size()) return SF_EINVAL;
  if (name && cap > 0) {
    std::strncpy(name, m->list[i].name.c_str(), cap - 1);
    name[cap - 1] = 0;
  }
  if (numel) *numel = m->list[i].numel();
  return SF_OK;
}

static void gen_one(const std::vector<sfh::TSpec>& list, uint64_t seed, bool full, int32_t i,
                    float* out) {
  std::vector<sfh::TSpec> one(list.size(), sfh::TSpec{"", {0}, 'b'});
  one[i] = list[i];
  std::vector<std::vector<float>> w;
  sfh::generate(one, seed, full, w);
  std::memcpy(out, w[i].data(), w[i].size() * 4);
}

sf_status sortformer_get_weights(const sf_model* m, int32_t i, float* host_out) {
  if (!m || !host_out || i < 0 || i >= (int32_t)m->list.size()) return SF_EINVAL;
  gen_one(m->list, m->seed, m->cfg.init_mode == SF_INIT_FULL_RANDOM, i, host_out);
  return SF_OK;
}

int32_t sortformer_config_num_tensors(const sf_model_config* c) {
  if (!valid_config(c)) return 0;
  return (int32_t)(c->arch == SF_ARCH_SORTFORMER ? sfh::sortformer_list(c->n_spk)
                                                 : sfh::nemotron_list(c->n_spk)).size();
}

sf_status sortformer_config_tensor(const sf_model_config* c, uint64_t seed, int32_t i, char* name,
                                   int32_t cap, int64_t* numel, float* host_out) {
  if (!valid_config(c)) return SF_EINVAL;
  const auto list = c->arch == SF_ARCH_SORTFORMER ? sfh::sortformer_list(c->n_spk)
                                                  : sfh::nemotron_list(c->n_spk);
  if (i < 0 || i >= (int32_t)list.size()) return SF_EINVAL;
  if (name && cap > 0) {
    std::strncpy(name, list[i].name.c_str(), cap - 1);
    name[cap - 1] = 0;
  }
  if (numel) *numel = list[i].numel();
  if (host_out) gen_one(list, seed, c->init_mode == SF_INIT_FULL_RANDOM, i, host_out);
  return SF_OK;
}

size_t sortformer_offline_workspace_bytes(const sf_model* m, int32_t B, int64_t N) {
  if (!m || B < 1 || N < 0) return 0;
  const int Te = frames_of(N);
  if (m->cfg.arch == SF_ARCH_SORTFORMER) {
    if (Te <= SF_MAX_WINDOW)
      return al256(enc_ws_bytes(m, B, std::max(Te, 1))) + al256(pre_ws_bytes(m, B, Te));
    sf_stream_config c{};  // longer clips: 'very high' chunks, pre-encoded per chunk
    sortformer_stream_preset("very_high", &c);
    return al256(pre_ws_bytes(m, B, c.chunk_len + c.right_context)) +
           al256(state_layout(m, &c, B).total) + al256(enc_ws_bytes(m, B, stream_cap(&c)));
  }
  sf_stream_config c{};
  sortformer_stream_preset("nemotron_offline", &c);
  return al256(pre_ws_bytes(m, B, Te)) + al256((size_t)B * (Te + 1) * 512 * 4) +
         al256(state_layout(m, &c, B).total) + al256(enc_ws_bytes(m, B, stream_cap(&c)));
}

sf_status sortformer_forward_offline(sf_model* m, const float* d_audio, int32_t B, int64_t N,
                                     float* d_probs, int64_t* n_out, void* d_ws, size_t ws_bytes,
                                     void* stream) {
  if (!m || !d_audio || !d_probs || !n_out || !d_ws || B < 1 || N < 0) return SF_EINVAL;
  const size_t need = sortformer_offline_workspace_bytes(m, B, N);
  if (need == 0) return SF_ESHAPE;
  if (ws_bytes < need) return SF_ENOMEM;
  const hipStream_t s = HS(stream);
  const int T = (int)(N / 160), Te = frames_of(N), S = m->cfg.n_spk;
  char* p = static_cast<char*>(d_ws);
  if (m->cfg.arch == SF_ARCH_SORTFORMER && Te > SF_MAX_WINDOW) {
    // longer than one encoder window: the 'very high' configuration's chunks
    // (340 frames + 40 look-ahead) with the speaker cache and FIFO, on the
    // known-length schedule; each chunk is pre-encoded from the clip when it
    // enters the window
    *n_out = Te;
    sf_stream st{};
    st.m = m;
    sortformer_stream_preset("very_high", &st.sc);
    st.B = B; st.S = S; st.D = 512;
    st.use_graphs = false;
    st.cap_stream = nullptr;
    st.cap = stream_cap(&st.sc);
    st.ring_cap = ring_cap_for(&st.sc);
    const int L = st.sc.chunk_len, R = st.sc.right_context;
    char* pre = p;
    p += al256(pre_ws_bytes(m, B, L + R));
    bind_state(&st, p);
    p += al256(state_layout(m, &st.sc, B).total);
    EncWs enc = carve_enc(m, p, B, st.cap);
    reset_host(&st);
    reset_device(&st, s);
    for (int c0 = 0; c0 < Te; c0 += L) {
      const int c1 = std::min(Te, c0 + L);
      const int rc = c1 == Te ? 0 : std::min(R, Te - c1);
      const int e1 = c1 + rc;
      pre_encode_range(m, d_audio, N, -1, N, T, st.enc_done, e1, B,
                       st.E[st.cur] + (size_t)(st.Lc + st.Lf + st.Lp) * 512,
                       (long long)st.cap * 512, pre, s);
      st.Lp += e1 - st.enc_done;
      st.enc_done = e1;
      step_core(&st, c1 - c0, d_probs + (size_t)c0 * S, (long long)Te * S, enc, nullptr, s);
    }
    return launched();
  }
  if (m->cfg.arch == SF_ARCH_SORTFORMER) {
    *n_out = Te;
    if (Te == 0) return SF_OK;
    EncWs enc = carve_enc(m, p, B, Te);
    char* pre = p + al256(enc_ws_bytes(m, B, Te));
    pre_encode_range(m, d_audio, N, -1, N, T, 0, Te, B, enc.x, (long long)Te * 512, pre, s);
    encode(m, enc, B, Te, Te, s);
    copy_rows(enc.probs, 0, S, d_probs, 0, S, 1, B * Te, S, s);
    return launched();
  }
  // Nemotron-style: 30.4 s chunks with the arrival-order cache and FIFO.
  const int per = 8 / m->out_stride;  // output frames per encoder frame
  *n_out = (long long)per * Te;
  if (Te == 0) return SF_OK;
  sf_stream st{};
  st.m = m;
  sortformer_stream_preset("nemotron_offline", &st.sc);
  st.B = B; st.S = S; st.D = 512;
  st.use_graphs = false;
  st.cap_stream = nullptr;
  st.cap = stream_cap(&st.sc);
  st.ring_cap = ring_cap_for(&st.sc);
  char* pre = p;
  p += al256(pre_ws_bytes(m, B, Te));
  float* emb = reinterpret_cast<float*>(p);
  p += al256((size_t)B * (Te + 1) * 512 * 4);
  bind_state(&st, p);
  p += al256(state_layout(m, &st.sc, B).total);
  EncWs enc = carve_enc(m, p, B, st.cap);
  reset_host(&st);
  reset_device(&st, s);
  pre_encode_range(m, d_audio, N, -1, N, T, 0, Te, B, emb, (long long)Te * 512, pre, s);
  const int L = st.sc.chunk_len, R = st.sc.right_context;
  for (int c0 = 0; c0 < Te; c0 += L) {
    const int c1 = std::min(Te, c0 + L);
    const int rc = c1 == Te ? 0 : std::min(R, Te - c1);
    const int e1 = c1 + rc;
    copy_rows(emb + (size_t)st.enc_done * 512, (long long)Te * 512, 512,
              st.E[st.cur] + (size_t)(st.Lc + st.Lf + st.Lp) * 512, (long long)st.cap * 512, 512, B,
              e1 - st.enc_done, 512, s);
    st.Lp += e1 - st.enc_done;
    st.enc_done = e1;
    step_core(&st, c1 - c0, d_probs + (size_t)per * c0 * S, (long long)per * Te * S, enc, nullptr,
              s);
  }
  return launched();
}

size_t sortformer_state_bytes(const sf_model* m, const sf_stream_config* c, int32_t B) {
  if (!m || !valid_stream_config(c) || B < 1 || stream_cap(c) > SF_MAX_WINDOW) return 0;
  return state_layout(m, c, B).total;
}

size_t sortformer_stream_workspace_bytes(const sf_model* m, const sf_stream_config* c, int32_t B) {
  if (!m || !valid_stream_config(c) || B < 1 || stream_cap(c) > SF_MAX_WINDOW) return 0;
  return stream_ws_bytes(m, c, B);
}

sf_status sortformer_stream_create(sf_model* m, const sf_stream_config* c, int32_t B,
                                   void* d_state, size_t bytes, void* stream, sf_stream** out) {
  if (!m || !valid_stream_config(c) || B < 1 || !d_state || !out) return SF_EINVAL;
  if (stream_cap(c) > SF_MAX_WINDOW) return SF_ESHAPE;
  if (c->spkcache_len / m->cfg.n_spk < 1) return SF_ESHAPE;
  if (reinterpret_cast<uintptr_t>(d_state) % 256) return SF_EINVAL;
  if (bytes < state_layout(m, c, B).total) return SF_ENOMEM;
  sf_stream* st = new (std::nothrow) sf_stream{};
  if (!st) return SF_ENOMEM;
  st->m = m;
  st->sc = *c;
  st->B = B;
  st->S = m->cfg.n_spk;
  st->D = 512;
  st->cap = stream_cap(c);
  st->ring_cap = ring_cap_for(c);
  st->use_graphs = true;
  st->fixed_window = false;
  st->cap_stream = nullptr;
  st->graph_ws = nullptr;
  bind_state(st, static_cast<char*>(d_state));
  reset_host(st);
  reset_device(st, HS(stream));
  if (launched() != SF_OK) {
    delete st;
    return SF_EHIP;
  }
  *out = st;
  return SF_OK;
}

void sortformer_stream_destroy(sf_stream* st) {
  if (!st) return;
  drop_graphs(st);
  if (st->cap_stream) (void)hipStreamDestroy(static_cast<hipStream_t>(st->cap_stream));
  delete st;
}

sf_status sortformer_stream_set_option(sf_stream* st, int32_t option, int32_t value) {
  if (!st) return SF_EINVAL;
  if (option == SF_STREAM_OPT_GRAPHS) {
    st->use_graphs = value != 0;
    if (!st->use_graphs) drop_graphs(st);
    return SF_OK;
  }
  if (option == SF_STREAM_OPT_FIXED_WINDOW) {
    if ((value != 0) != st->fixed_window) drop_graphs(st);  // keys change meaning
    st->fixed_window = value != 0;
    return SF_OK;
  }
  return SF_EINVAL;
}

sf_status sortformer_stream_reset(sf_stream* st, void* stream) {
  if (!st) return SF_EINVAL;
  reset_host(st);
  reset_device(st, HS(stream));
  return launched();
}

int64_t sortformer_stream_samples_needed(const sf_stream* st) {
  if (!st) return -1;
  if (st->finished) return 0;
  if (st->steps == 0) return 1280LL * (st->sc.chunk_len + st->sc.right_context) + 40;
  return 1280LL * st->sc.chunk_len;
}

int32_t sortformer_stream_max_emit(const sf_stream* st) {
  if (!st) return 0;
  const int n = st->sc.chunk_len + st->sc.right_context;
  return st->m->cfg.arch == SF_ARCH_NEMOTRON ? 8 / st->m->out_stride * n : n;
}

sf_status sortformer_set_option(sf_model* m, int32_t option, int32_t value) {
  if (!m) return SF_EINVAL;
  if (option == SF_OPT_OUTPUT_STRIDE) {
    if (value != 1 && value != 2 && value != 4 && value != 8) return SF_EINVAL;
    if (m->cfg.arch != SF_ARCH_NEMOTRON && value != 1) return SF_EUNSUPPORTED;
    m->out_stride = value;
    return SF_OK;
  }
  return SF_EINVAL;
}

int32_t sortformer_get_option(const sf_model* m, int32_t option) {
  if (!m) return -1;
  return option == SF_OPT_OUTPUT_STRIDE ? m->out_stride : -1;
}

}  // extern "C"

namespace {
// Host arithmetic of the next step of a stream whose samples [recv, recv +
// n_new) are (or are about to be) in the audio ring: the encoder frames it
// pre-encodes (up to e1), the rows it scores (n_chunk) and its window W. The
// non-final step s covers frames up to (s+1)*chunk_len + right_context; the
// final one scores every remaining frame of the clip with no look-ahead
// (Transformers docs "Nemotron 3 Diarization", streaming usage). Returns false
// when the counters are inconsistent or the window would not fit the state.
struct StepPlan {
  long long N;
  int e1, n_chunk, W;
};
bool plan_step(const sf_stream* st, long long n_new, bool is_last, StepPlan* p) {
  const int L = st->sc.chunk_len, R = st->sc.right_context;
  p->N = st->recv + n_new;
  const long long e1 = is_last ? frames_of(p->N) : (st->steps + 1) * L + R;
  if (e1 > INT_MAX / 2 || e1 < st->enc_done) return false;
  p->e1 = (int)e1;
  const long long n_chunk = is_last ? e1 - st->emitted : L;
  const int fresh = p->e1 - st->enc_done;
  if (n_chunk < 0 || n_chunk > st->Lp + fresh) return false;
  p->n_chunk = (int)n_chunk;
  p->W = st->Lc + st->Lf + st->Lp + fresh;
  return p->W <= st->cap;
}

// One step whose new samples are already in the ring: pre-encode the new
// frames into the look-ahead rows, run the window, emit the chunk rows to
// out (row stride S, batch stride out_bstride floats) and update the cache.
// graphs: the window forward may run from a captured graph (stream option).
void step_from_ring(sf_stream* st, const StepPlan& p, bool is_last, float* out,
                    long long out_bstride, void* d_ws, hipStream_t s, bool graphs = true) {
  char* ws = static_cast<char*>(d_ws);
  EncWs enc = carve_enc(st->m, ws, st->B, st->cap);
  char* pre = ws + al256(enc_ws_bytes(st->m, st->B, st->cap));
  const int T = (int)(p.N / 160);
  pre_encode_range(st->m, st->ring, st->ring_cap, st->ring_cap - 1, p.N, T, st->enc_done, p.e1,
                   st->B, st->E[st->cur] + (size_t)(st->Lc + st->Lf + st->Lp) * st->D,
                   (long long)st->cap * st->D, pre, s);
  st->Lp += p.e1 - st->enc_done;
  st->enc_done = p.e1;
  st->recv = p.N;
  if (p.n_chunk > 0) step_core(st, p.n_chunk, out, out_bstride, enc, graphs ? d_ws : nullptr, s);
  st->steps += 1;
  st->emitted += p.n_chunk;
  st->finished = is_last;
}

int emit_rate(const sf_stream* st) {
  return st->m->cfg.arch == SF_ARCH_NEMOTRON ? 8 / st->m->out_stride : 1;
}

// The steps a feed of n_new more samples runs, on a copy of the counters: the
// non-final steps whose audio is complete, then (is_last) the final step.
// Returns false if any of them would be refused.
bool plan_feed(const sf_stream* st0, long long n_new, bool is_last, long long* frames,
               int* n_steps) {
  sf_stream st = *st0;  // host counters only; no device work
  st.graphs.clear();
  long long avail = st.pending + n_new, out = 0;
  int k = 0;
  while (!st.finished) {
    const long long need = sortformer_stream_samples_needed(&st);
    const bool full = avail >= need;
    if (!full && !is_last) break;
    StepPlan p;
    if (!plan_step(&st, full ? need : avail, !full, &p)) return false;
    const Lens n = lens_after_update(st.sc, st.Lc, st.Lf, st.Lp + p.e1 - st.enc_done, p.n_chunk);
    st.Lc = n.Lc; st.Lf = n.Lf; st.Lp = n.Lp;
    st.enc_done = p.e1;
    st.recv = p.N;
    st.steps += 1;
    st.emitted += p.n_chunk;
    st.finished = !full;
    avail -= full ? need : avail;
    out += (long long)emit_rate(&st) * p.n_chunk;
    ++k;
  }
  *frames = out;
  *n_steps = k;
  return true;
}

// Checkpoint blob: a fixed header, then emb (B, rows, D) fp32, probs (B, rows,
// S) fp32, flags (B, rows) int32, silence sums (B, D) fp64, silence counts (B)
// int32 and the audio ring (B, ring_cap) fp32, each section 256-byte aligned
// and sized for the capacity (rows = cache + FIFO + look-ahead rows in use,
// stored densely at the start of their section), so every blob of a stream
// configuration has the same size.
constexpr uint64_t CKPT_MAGIC = 0x3130544b43464653ull;  // "SFFCKT01"
struct CkptHeader {
  uint64_t magic;
  int32_t version, arch, n_spk, dim, batch, cap;
  int32_t cfg[6];
  int64_t ring_cap;
  int32_t Lc, Lf, Lp, enc_done;
  int64_t steps, emitted, recv, pending;
  int32_t finished, rows;
  int64_t bytes;
};
static_assert(sizeof(CkptHeader) <= 256, "checkpoint header");
struct CkptLayout {
  size_t emb, probs, flags, sum, cnt, ring, total;
};
CkptLayout ckpt_layout(int B, int rows, int D, int S, long long ring_cap) {
  CkptLayout c{};
  size_t o = 256;
  c.emb = o; o += al256((size_t)B * rows * D * 4);
  c.probs = o; o += al256((size_t)B * rows * S * 4);
  c.flags = o; o += al256((size_t)B * rows * 4);
  c.sum = o; o += al256((size_t)B * D * 8);
  c.cnt = o; o += al256((size_t)B * 4);
  c.ring = o; o += al256((size_t)B * ring_cap * 4);
  c.total = o;
  return c;
}

// Rows [0, rows) of the current state buffers <-> host (row-major, dense).
bool copy_rows_host(sf_stream* st, bool to_host, int rows, float* emb, float* probs, int32_t* flags,
                    double* sum, int32_t* cnt, hipStream_t s) {
  const int B = st->B, D = st->D, S = st->S, cur = st->cur;
  const hipMemcpyKind k = to_host ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice;
  auto c2 = [&](void* dev, void* host, size_t row_bytes, size_t dev_pitch) -> bool {
    if (rows == 0 || !host) return true;
    void* dst = to_host ? host : dev;
    const void* src = to_host ? dev : host;
    const size_t dp = to_host ? row_bytes * rows : dev_pitch, sp = to_host ? dev_pitch : row_bytes * rows;
    return hipMemcpy2DAsync(dst, dp, src, sp, row_bytes * rows, B, k, s) == hipSuccess;
  };
  bool ok = c2(st->E[cur], emb, (size_t)D * 4, (size_t)st->cap * D * 4) &&
            c2(st->P[cur], probs, (size_t)S * 4, (size_t)st->cap * S * 4) &&
            c2(st->ph[cur], flags, 4, (size_t)st->cap * 4);
  if (ok && sum)
    ok = (to_host ? hipMemcpyAsync(sum, st->sil_sum, (size_t)B * D * 8, k, s)
                  : hipMemcpyAsync(st->sil_sum, sum, (size_t)B * D * 8, k, s)) == hipSuccess;
  if (ok && cnt)
    ok = (to_host ? hipMemcpyAsync(cnt, st->sil_cnt, (size_t)B * 4, k, s)
                  : hipMemcpyAsync(st->sil_cnt, cnt, (size_t)B * 4, k, s)) == hipSuccess;
  return ok;
}
}  // namespace

extern "C" {

sf_status sortformer_stream_step(sf_stream* st, const float* d_audio_new, int64_t n_new,
                                 int32_t is_last, float* d_probs_out, int32_t* n_emitted,
                                 void* d_ws, size_t ws_bytes, void* stream) {
  if (!st || !n_emitted || !d_ws || !d_probs_out) return SF_EINVAL;
  if (st->finished || st->rows_only || st->pending != 0) return SF_ESTATE;
  const long long need = sortformer_stream_samples_needed(st);
  if (n_new < 0 || n_new > need || (!is_last && n_new != need)) return SF_ESHAPE;
  if (n_new > 0 && !d_audio_new) return SF_EINVAL;
  if (ws_bytes < stream_ws_bytes(st->m, &st->sc, st->B)) return SF_ENOMEM;
  StepPlan p;
  if (!plan_step(st, n_new, is_last != 0, &p)) return SF_ESTATE;
  const hipStream_t s = HS(stream);
  *n_emitted = emit_rate(st) * p.n_chunk;
  ring_write(d_audio_new, n_new, n_new, st->B, st->ring, st->ring_cap, st->recv, s);
  step_from_ring(st, p, is_last != 0, d_probs_out, (long long)(*n_emitted) * st->S, d_ws, s);
  return launched();
}

int64_t sortformer_stream_feed_frames(const sf_stream* st, int64_t n_new, int32_t is_last) {
  if (!st || n_new < 0 || st->rows_only) return -1;
  if (st->finished) return n_new == 0 ? 0 : -1;
  long long frames = 0;
  int k = 0;
  if (!plan_feed(st, n_new, is_last != 0, &frames, &k)) return -1;
  return frames;
}

sf_status sortformer_stream_feed(sf_stream* st, const float* d_audio_new, int64_t n_new,
                                 int32_t is_last, float* d_probs_out, int64_t out_frames,
                                 int64_t* n_emitted, void* d_ws, size_t ws_bytes, void* stream) {
  if (!st || !n_emitted || !d_ws || n_new < 0) return SF_EINVAL;
  if (n_new > 0 && !d_audio_new) return SF_EINVAL;
  if (st->finished || st->rows_only) return SF_ESTATE;
  if (ws_bytes < stream_ws_bytes(st->m, &st->sc, st->B)) return SF_ENOMEM;
  long long frames = 0;
  int n_steps = 0;
  if (!plan_feed(st, n_new, is_last != 0, &frames, &n_steps)) return SF_ESTATE;
  if (frames > out_frames || (frames > 0 && !d_probs_out)) return SF_ENOMEM;
  *n_emitted = frames;
  const hipStream_t s = HS(stream);
  const long long ob = out_frames * st->S;  // batch stride of the output (floats)
  long long used = 0, e0 = 0;               // samples of d_audio_new consumed, frames emitted
  for (int i = 0; i < n_steps; ++i) {
    const long long need = sortformer_stream_samples_needed(st);
    const long long take = std::min(need - st->pending, n_new - used);
    ring_write(d_audio_new + used, n_new, take, st->B, st->ring, st->ring_cap,
               st->recv + st->pending, s);
    used += take;
    const bool full = st->pending + take >= need;
    StepPlan p;
    plan_step(st, st->pending + take, !full, &p);  // checked by plan_feed
    st->pending = 0;
    step_from_ring(st, p, !full, d_probs_out + e0 * st->S, ob, d_ws, s);
    e0 += (long long)emit_rate(st) * p.n_chunk;
  }
  // the rest waits in the ring for the next feed
  ring_write(d_audio_new + used, n_new, n_new - used, st->B, st->ring, st->ring_cap,
             st->recv + st->pending, s);
  st->pending += n_new - used;
  return launched();
}

}  // extern "C"

namespace {
// Step workspace for callers that cannot allocate: one static device array per
// GPU, of SF_NOALLOC_SCRATCH_BYTES, alive until the process ends. Its address
// on each device is taken once, with that device current; host code uses only
// that address (the array's own name is a host-side stand-in).
static __device__ __align__(256) char scratch[SF_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

sf_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SF_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SF_EHIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return SF_OK;
}
}  // namespace

extern "C" {

sf_status sortformer_stream_step_noalloc(sf_stream* st, const float* d_audio_new, int64_t n_new,
                                         int32_t is_last, float* d_probs_out,
                                         int32_t* n_emitted, void* stream) {
  if (!st || !n_emitted || !d_probs_out) return SF_EINVAL;
  if (st->finished || st->rows_only || st->pending != 0) return SF_ESTATE;
  const long long need = sortformer_stream_samples_needed(st);
  if (n_new < 0 || n_new > need || (!is_last && n_new != need)) return SF_ESHAPE;
  if (n_new > 0 && !d_audio_new) return SF_EINVAL;
  const size_t ws_bytes = stream_ws_bytes(st->m, &st->sc, st->B);
  if (ws_bytes > SF_NOALLOC_SCRATCH_BYTES) return SF_ENOMEM;  // beyond the static scratch
  StepPlan p;
  if (!plan_step(st, n_new, is_last != 0, &p)) return SF_ESTATE;
  void* ws = nullptr;
  const sf_status got = scratch_on_current_device(&ws);
  if (got != SF_OK) return got;
  const hipStream_t s = HS(stream);
  *n_emitted = emit_rate(st) * p.n_chunk;
  ring_write(d_audio_new, n_new, n_new, st->B, st->ring, st->ring_cap, st->recv, s);
  step_from_ring(st, p, is_last != 0, d_probs_out, (long long)(*n_emitted) * st->S, ws, s, false);
  return launched();
}

sf_status sortformer_stream_get_info(const sf_stream* st, int64_t* info, void** ptrs) {
  if (!st) return SF_EINVAL;
  if (info) {
    info[0] = st->Lc; info[1] = st->Lf; info[2] = st->Lp; info[3] = st->cap;
    info[4] = st->steps; info[5] = st->emitted; info[6] = st->recv; info[7] = st->finished;
    info[8] = st->pending;
  }
  if (ptrs) {
    ptrs[0] = st->E[st->cur]; ptrs[1] = st->P[st->cur]; ptrs[2] = st->ph[st->cur];
    ptrs[3] = st->sil_sum; ptrs[4] = st->sil_cnt;
    ptrs[5] = reinterpret_cast<void*>((intptr_t)st->D);
  }
  return SF_OK;
}

sf_status sortformer_stream_get_rows(const sf_stream* st, float* emb, float* probs, int32_t* flags,
                                     double* sum, int32_t* cnt, void* stream) {
  if (!st) return SF_EINVAL;
  sf_stream* m = const_cast<sf_stream*>(st);
  const hipStream_t s = HS(stream);
  if (!copy_rows_host(m, true, st->Lc + st->Lf + st->Lp, emb, probs, flags, sum, cnt, s) ||
      hipStreamSynchronize(s) != hipSuccess)
    return SF_EHIP;
  return SF_OK;
}

sf_status sortformer_stream_set_rows(sf_stream* st, int32_t Lc, int32_t Lf, int32_t Lp,
                                     const float* emb, const float* probs, const int32_t* flags,
                                     const double* sum, const int32_t* cnt, void* stream) {
  if (!st) return SF_EINVAL;
  if (Lc < 0 || Lf < 0 || Lp < 0 || Lc > st->sc.spkcache_len || Lf > st->sc.fifo_len ||
      Lp > st->sc.chunk_len + st->sc.right_context)
    return SF_ESHAPE;
  if ((Lc + Lf + Lp > 0) && (!emb || !probs || !flags)) return SF_EINVAL;
  const hipStream_t s = HS(stream);
  if (!copy_rows_host(st, false, Lc + Lf + Lp, const_cast<float*>(emb), const_cast<float*>(probs),
                      const_cast<int32_t*>(flags), const_cast<double*>(sum),
                      const_cast<int32_t*>(cnt), s) ||
      hipStreamSynchronize(s) != hipSuccess)
    return SF_EHIP;
  st->Lc = Lc; st->Lf = Lf; st->Lp = Lp;
  st->rows_only = true;
  return SF_OK;
}

size_t sortformer_stream_checkpoint_bytes(const sf_stream* st) {
  if (!st) return 0;
  return ckpt_layout(st->B, st->cap, st->D, st->S, st->ring_cap).total;
}

sf_status sortformer_stream_export(const sf_stream* st, void* host, size_t bytes, void* stream) {
  if (!st || !host) return SF_EINVAL;
  if (st->rows_only) return SF_ESTATE;
  if (bytes < sortformer_stream_checkpoint_bytes(st)) return SF_ENOMEM;
  const int rows = st->Lc + st->Lf + st->Lp;
  const CkptLayout L = ckpt_layout(st->B, st->cap, st->D, st->S, st->ring_cap);
  char* h = static_cast<char*>(host);
  std::memset(h, 0, L.total);
  CkptHeader hd{};
  hd.magic = CKPT_MAGIC;
  hd.version = 1;
  hd.arch = st->m->cfg.arch; hd.n_spk = st->S; hd.dim = st->D; hd.batch = st->B; hd.cap = st->cap;
  const sf_stream_config& c = st->sc;
  const int32_t cfg[6] = {c.chunk_len, c.right_context, c.fifo_len, c.update_period,
                          c.spkcache_len, c.n_sil_per_spk};
  std::memcpy(hd.cfg, cfg, sizeof cfg);
  hd.ring_cap = st->ring_cap;
  hd.Lc = st->Lc; hd.Lf = st->Lf; hd.Lp = st->Lp; hd.enc_done = st->enc_done;
  hd.steps = st->steps; hd.emitted = st->emitted; hd.recv = st->recv; hd.pending = st->pending;
  hd.finished = st->finished; hd.rows = rows;
  hd.bytes = (int64_t)L.total;
  std::memcpy(h, &hd, sizeof hd);
  sf_stream* m = const_cast<sf_stream*>(st);
  const hipStream_t s = HS(stream);
  bool ok = copy_rows_host(m, true, rows, reinterpret_cast<float*>(h + L.emb),
                           reinterpret_cast<float*>(h + L.probs), reinterpret_cast<int32_t*>(h + L.flags),
                           reinterpret_cast<double*>(h + L.sum), reinterpret_cast<int32_t*>(h + L.cnt), s);
  ok = ok && hipMemcpyAsync(h + L.ring, st->ring, (size_t)st->B * st->ring_cap * 4,
                            hipMemcpyDeviceToHost, s) == hipSuccess;
  if (!ok || hipStreamSynchronize(s) != hipSuccess) return SF_EHIP;
  return SF_OK;
}

sf_status sortformer_stream_import(sf_stream* st, const void* host, size_t bytes, void* stream) {
  if (!st || !host || bytes < 256) return SF_EINVAL;
  CkptHeader hd;
  std::memcpy(&hd, host, sizeof hd);
  const sf_stream_config& c = st->sc;
  const int32_t cfg[6] = {c.chunk_len, c.right_context, c.fifo_len, c.update_period,
                          c.spkcache_len, c.n_sil_per_spk};
  if (hd.magic != CKPT_MAGIC || hd.version != 1) return SF_EINVAL;
  if (hd.arch != st->m->cfg.arch || hd.n_spk != st->S || hd.dim != st->D || hd.batch != st->B ||
      hd.cap != st->cap || hd.ring_cap != st->ring_cap || std::memcmp(hd.cfg, cfg, sizeof cfg) != 0)
    return SF_EINVAL;  // another model, batch or stream configuration
  // counters of a stream the step/feed functions produced: lengths within the
  // configuration, the look-ahead rows are the pre-encoded frames not yet
  // scored, cache + FIFO hold at most the scored frames, the samples held
  // cover every pre-encoded frame and less than one step is pending
  const bool sane =
      hd.rows == hd.Lc + hd.Lf + hd.Lp && hd.Lc >= 0 && hd.Lf >= 0 && hd.Lp >= 0 &&
      hd.Lc <= c.spkcache_len && hd.Lf <= c.fifo_len && hd.Lp <= c.chunk_len + c.right_context &&
      hd.steps >= 0 && hd.emitted >= 0 && hd.recv >= 0 && hd.pending >= 0 && hd.enc_done >= 0 &&
      (hd.finished == 0 || hd.finished == 1) && hd.emitted + hd.Lp == hd.enc_done &&
      hd.Lc + hd.Lf <= hd.emitted && hd.enc_done <= frames_of(hd.recv) &&
      hd.pending < 1280LL * (c.chunk_len + c.right_context) + 40 &&
      (hd.steps > 0 || (hd.recv == 0 && hd.enc_done == 0));
  if (!sane) return SF_EINVAL;
  const CkptLayout L = ckpt_layout(st->B, st->cap, st->D, st->S, st->ring_cap);
  if (hd.bytes != (int64_t)L.total || bytes < L.total) return SF_EINVAL;
  const char* h = static_cast<const char*>(host);
  const hipStream_t s = HS(stream);
  reset_device(st, s);  // flags of both buffers cleared
  st->cur = 0;
  bool ok = copy_rows_host(st, false, hd.rows, reinterpret_cast<float*>(const_cast<char*>(h + L.emb)),
                           reinterpret_cast<float*>(const_cast<char*>(h + L.probs)),
                           reinterpret_cast<int32_t*>(const_cast<char*>(h + L.flags)),
                           reinterpret_cast<double*>(const_cast<char*>(h + L.sum)),
                           reinterpret_cast<int32_t*>(const_cast<char*>(h + L.cnt)), s);
  ok = ok && hipMemcpyAsync(st->ring, h + L.ring, (size_t)st->B * st->ring_cap * 4,
                            hipMemcpyHostToDevice, s) == hipSuccess;
  if (!ok || hipStreamSynchronize(s) != hipSuccess) {
    reset_host(st);  // never leave half-imported counters behind
    return SF_EHIP;
  }
  st->Lc = hd.Lc; st->Lf = hd.Lf; st->Lp = hd.Lp; st->enc_done = hd.enc_done;
  st->steps = hd.steps; st->emitted = hd.emitted; st->recv = hd.recv; st->pending = hd.pending;
  st->finished = hd.finished != 0;
  st->rows_only = false;
  return SF_OK;
}

sf_status sortformer_stream_update(sf_stream* st, const float* d_wp, int32_t n_chunk, void* d_ws,
                                   size_t ws_bytes, void* stream) {
  if (!st || !d_wp || !d_ws) return SF_EINVAL;
  if (n_chunk < 0 || n_chunk > st->Lp) return SF_ESHAPE;
  if (ws_bytes < stream_ws_bytes(st->m, &st->sc, st->B)) return SF_ENOMEM;
  const hipStream_t s = HS(stream);
  const int W = st->Lc + st->Lf + st->Lp;
  EncWs enc = carve_enc(st->m, static_cast<char*>(d_ws), st->B, st->cap);
  copy_rows(d_wp, 0, st->S, enc.probs, 0, st->S, 1, st->B * W, st->S, s);
  state_update(st, enc.probs, W, n_chunk, s);
  return launched();
}

size_t sortformer_encode_workspace_bytes(const sf_model* m, int32_t B, int32_t W) {
  if (!m || B < 1 || W < 1 || W > SF_MAX_WINDOW) return 0;
  return enc_ws_bytes(m, B, W);
}

sf_status sortformer_encode_window(sf_model* m, const float* d_emb, int32_t B, int32_t W,
                                   int32_t n_valid, float* d_probs, float* d_probs10, void* d_ws,
                                   size_t ws_bytes, void* stream) {
  if (!m || !d_emb || !d_probs || !d_ws) return SF_EINVAL;
  if (B < 1 || W < 1 || W > SF_MAX_WINDOW || n_valid < 1 || n_valid > W) return SF_ESHAPE;
  if (ws_bytes < enc_ws_bytes(m, B, W)) return SF_ENOMEM;
  const hipStream_t s = HS(stream);
  const int S = m->cfg.n_spk;
  for (const auto& t : m->taps)
    if (t.cap < (size_t)B * W * tap_width(m, t.layer)) return SF_ENOMEM;
  EncWs enc = carve_enc(m, static_cast<char*>(d_ws), B, W);
  copy_rows(d_emb, 0, 512, enc.x, 0, 512, 1, B * W, 512, s);
  encode(m, enc, B, W, n_valid, s, true);
  copy_rows(enc.probs, 0, S, d_probs, 0, S, 1, B * W, S, s);
  if (d_probs10 && m->cfg.arch == SF_ARCH_NEMOTRON)
    copy_rows(enc.probs10, 0, S, d_probs10, 0, S, 1, B * W * 8, S, s);
  return launched();
}

sf_status sortformer_debug_tap(sf_model* m, int32_t layer, int32_t point, float* d_out,
                               size_t out_floats) {
  if (!m) return SF_EINVAL;
  if (layer == -1 && !d_out) {
    m->taps.clear();
    return SF_OK;
  }
  if (point < SF_TAP_LAYER_IN || point > SF_TAP_LAYER_OUT) return SF_EINVAL;
  if (layer < 0 || layer >= tap_layers(m)) return SF_ESHAPE;
  auto it = m->taps.begin();
  while (it != m->taps.end() && !(it->layer == layer && it->point == point)) ++it;
  if (!d_out) {
    if (it != m->taps.end()) m->taps.erase(it);
    return SF_OK;
  }
  if (it != m->taps.end()) {
    it->out = d_out;
    it->cap = out_floats;
    return SF_OK;
  }
  if (m->taps.size() >= SF_MAX_TAPS) return SF_EINVAL;
  m->taps.push_back({layer, point, d_out, out_floats});
  return SF_OK;
}

size_t sortformer_pre_encode_workspace_bytes(const sf_model* m, int32_t B, int64_t N) {
  if (!m || B < 1 || N < 0) return 0;
  const int Te = frames_of(N);
  return al256(pre_ws_bytes(m, B, Te)) + al256((size_t)B * (Te + 1) * 512 * 4);
}

sf_status sortformer_pre_encode(sf_model* m, const float* d_audio, int32_t B, int64_t N,
                                float* d_mel, float* d_emb, void* d_ws, size_t ws_bytes,
                                void* stream) {
  if (!m || !d_audio || !d_ws || B < 1 || N < 0) return SF_EINVAL;
  const int T = (int)(N / 160), Te = frames_of(N);
  if (ws_bytes < sortformer_pre_encode_workspace_bytes(m, B, N)) return SF_ENOMEM;
  if (Te == 0) return SF_OK;
  const hipStream_t s = HS(stream);
  char* pre = static_cast<char*>(d_ws);
  float* emb = reinterpret_cast<float*>(pre + al256(pre_ws_bytes(m, B, Te)));
  pre_encode_range(m, d_audio, N, -1, N, T, 0, Te, B, emb, (long long)Te * 512, pre, s);
  if (d_mel) copy_rows(reinterpret_cast<float*>(pre), 0, 128, d_mel, 0, 128, 1, B * T, 128, s);
  if (d_emb) copy_rows(emb, 0, 512, d_emb, 0, 512, 1, B * Te, 512, s);
  return launched();
}

sf_status sortformer_profile_begin(int32_t cls, int32_t max_launches) {
  if (cls < PROF_GEMM || cls > PROF_CACHE || max_launches < 1) return SF_EINVAL;
  const int r = prof_start(cls, max_launches);
  return r == 0 ? SF_OK : (r == -1 ? SF_ESTATE : SF_EHIP);
}

sf_status sortformer_profile_end(double* ms, int64_t* launches, double* flops, double* bytes) {
  long long n = 0;
  const int r = prof_stop(ms, &n, flops, bytes);
  if (launches) *launches = n;
  return r == 0 ? SF_OK : (r == -5 ? SF_ESTATE : SF_EHIP);
}

// ------------------------------------------------------------------ segments
void sortformer_segment_defaults(sf_segment_params* out) {
  if (out) *out = sf_segment_params{0.5f, 0.5f, 0.0, 0.0, 0.0, 0.0};
}

int64_t sortformer_segments_capacity(int64_t n_frames) {
  return n_frames < 0 ? 0 : (n_frames + 1) / 2;
}

sf_status sortformer_segments(const float* d_probs, int32_t batch, int64_t n_frames,
                              int32_t n_spk, double frame_s, const sf_segment_params* params,
                              sf_segment* d_out, int64_t capacity, int64_t* d_counts,
                              void* stream) {
  if (!d_probs || !d_out || !d_counts || batch < 1 || n_frames < 0 || n_spk < 1 || n_spk > 64 ||
      !(frame_s > 0.0) || !std::isfinite(frame_s))
    return SF_EINVAL;
  if (n_frames > (int64_t)INT32_MAX || (int64_t)batch * n_spk > (int64_t)INT32_MAX) return SF_ESHAPE;
  sf_segment_params p;
  sortformer_segment_defaults(&p);
  if (params) p = *params;
  const bool ok = std::isfinite(p.onset) && std::isfinite(p.offset) && p.onset >= p.offset &&
                  p.pad_onset >= 0.0 && p.pad_offset >= 0.0 && p.min_duration_on >= 0.0 &&
                  p.min_duration_off >= 0.0 && std::isfinite(p.pad_onset) &&
                  std::isfinite(p.pad_offset) && std::isfinite(p.min_duration_on) &&
                  std::isfinite(p.min_duration_off);
  if (!ok) return SF_EINVAL;
  if (capacity < sortformer_segments_capacity(n_frames)) return SF_ENOMEM;
  sf::segments(d_probs, batch, (int)n_frames, n_spk, frame_s, p, d_out, capacity,
               reinterpret_cast<long long*>(d_counts), HS(stream));
  return launched();
}

}  // extern "C"
