// Model construction (weight arena, derived tables) and the forward graphs:
// frontend + pre_encode, the Sortformer encoder (17 conformer layers,
// projection, 18 post-LN transformer layers, speaker head) and the
// Nemotron-style encoder (31 pre-LN RoPE layers, upsampling head).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "host.h"
#include "kernels.h"
#include "model.h"

using namespace sf;
using namespace sfh;

namespace sfm {

// ------------------------------------------------------------------ arena
namespace {
struct Arena {
  size_t off = 0;
  char* dev = nullptr;   // device base (null while sizing)
  char* host = nullptr;  // staging copy of the arena (null while sizing)
  size_t alloc(size_t bytes) {
    const size_t o = (off + 255) & ~(size_t)255;
    off = o + bytes;
    return o;
  }
  const float* f32(const float* src, size_t n) {
    const size_t o = alloc(n * 4);
    if (host && src) std::memcpy(host + o, src, n * 4);
    return reinterpret_cast<const float*>(dev + o);
  }
  const void* act(const float* src, size_t n, bool bf16) {
    const size_t o = alloc(n * (bf16 ? 2 : 4));
    if (host && src) {
      if (bf16) {
        uint16_t* d = reinterpret_cast<uint16_t*>(host + o);
        for (size_t i = 0; i < n; ++i) {
          uint32_t u;
          std::memcpy(&u, &src[i], 4);
          u += 0x7FFFu + ((u >> 16) & 1u);
          d[i] = (uint16_t)(u >> 16);
        }
      } else {
        std::memcpy(host + o, src, n * 4);
      }
    }
    return dev + o;
  }
  // bf16 copy of an N x K row-major matrix in MFMA fragment-major order: 1 KB
  // block (t, s) = t * (K/32) + s holds rows 16t..16t+15, columns
  // 32s..32s+31, lane l = 16 g + c's 8 values W[16t + c][32s + 8g + e] at
  // element 8 l + e
  const void* frag(const float* src, int N, int K) {
    const size_t o = alloc((size_t)N * K * 2);
    if (host && src) {
      uint16_t* d = reinterpret_cast<uint16_t*>(host + o);
      for (int t = 0; t < N / 16; ++t)
        for (int sb = 0; sb < K / 32; ++sb)
          for (int l = 0; l < 64; ++l)
            for (int e = 0; e < 8; ++e) {
              const float f = src[(size_t)(16 * t + l % 16) * K + 32 * sb + 8 * (l / 16) + e];
              uint32_t u;
              std::memcpy(&u, &f, 4);
              u += 0x7FFFu + ((u >> 16) & 1u);
              d[((size_t)t * (K / 32) + sb) * 512 + 8 * l + e] = (uint16_t)(u >> 16);
            }
    }
    return dev + o;
  }
  void* raw(size_t bytes) { return dev + alloc(bytes); }
};

struct Src {
  const std::vector<TSpec>* list;
  const std::vector<std::vector<float>>* w;  // null while sizing
  const float* get(const std::string& n) const {
    if (!w) return nullptr;
    for (size_t i = 0; i < list->size(); ++i)
      if ((*list)[i].name == n) return (*w)[i].data();
    return nullptr;
  }
};

// Slaney mel filterbank (128 bands over 0-8 kHz, 257 bins of 31.25 Hz, area
// normalised), stored sparse: per band the first non-zero bin, the count and
// the weights.
double hz2mel(double f) { return f < 1000.0 ? 3.0 * f / 200.0 : 15.0 + 27.0 * std::log(f / 1000.0) / std::log(6.4); }
double mel2hz(double m) { return m < 15.0 ? 200.0 * m / 3.0 : 1000.0 * std::exp((m - 15.0) * std::log(6.4) / 27.0); }

std::vector<float> frontend_table() {
  std::vector<float> t(1680 + 128 * 32, 0.f);
  for (int m = 0; m < 512; ++m) {
    t[m] = (float)std::cos(2.0 * M_PI * m / 512.0);
    t[512 + m] = (float)std::sin(2.0 * M_PI * m / 512.0);
  }
  for (int n = 0; n < 400; ++n) t[1024 + n] = (float)(0.5 - 0.5 * std::cos(2.0 * M_PI * n / 400.0));
  double edges[130];
  const double mmax = hz2mel(8000.0);
  for (int i = 0; i < 130; ++i) edges[i] = mel2hz(mmax * i / 129.0);
  for (int m = 0; m < 128; ++m) {
    const double lo = edges[m], ce = edges[m + 1], hi = edges[m + 2];
    int first = -1, cnt = 0;
    for (int k = 0; k <= 256; ++k) {
      const double f = k * 31.25;
      const double wv = std::fmax(0.0, std::fmin((f - lo) / (ce - lo), (hi - f) / (hi - ce))) *
                        (2.0 / (hi - lo));
      if (wv > 0.0) {
        if (first < 0) first = k;
        const int i = k - first;
        if (i < 32) t[1680 + m * 32 + i] = (float)wv;
        cnt = i + 1;
      }
    }
    if (first < 0) first = 0;
    t[1424 + 2 * m] = (float)first;
    t[1424 + 2 * m + 1] = (float)(cnt > 32 ? 32 : cnt);
  }
  return t;
}

void build_sortformer(sf_model* m, Arena& A, const Src& s) {
  const bool bf = m->bf16;
  const bool have = s.w != nullptr;
  m->c0_w = A.f32(s.get("pre.conv0.w"), 256 * 9);
  m->c0_b = A.f32(s.get("pre.conv0.b"), 256);
  for (int k = 0; k < 2; ++k) {
    const std::string d = "pre.dw" + std::to_string(k + 1), p = "pre.pw" + std::to_string(k + 1);
    m->dw_w[k] = A.f32(s.get(d + ".w"), 256 * 9);
    m->dw_b[k] = A.f32(s.get(d + ".b"), 256);
    m->pw_w[k] = A.act(s.get(p + ".w"), 256 * 256, bf);
    m->pw_b[k] = A.f32(s.get(p + ".b"), 256);
  }
  {  // flatten order: channels-last rows give feature f*256+c; the card's is c*16+f
    std::vector<float> w;
    if (have) {
      const float* src = s.get("pre.out.w");
      w.resize(512 * 4096);
      for (int n = 0; n < 512; ++n)
        for (int c = 0; c < 256; ++c)
          for (int f = 0; f < 16; ++f) w[(size_t)n * 4096 + f * 256 + c] = src[(size_t)n * 4096 + c * 16 + f];
    }
    m->pre_out_w = A.act(have ? w.data() : nullptr, 512 * 4096, bf);
    m->pre_out_b = A.f32(s.get("pre.out.b"), 512);
  }
  for (int l = 0; l < 17; ++l) {
    const std::string p = "conf" + std::to_string(l) + ".";
    ConfLayer& L = m->conf[l];
    L.ff1_g = A.f32(s.get(p + "ff1.ln.g"), 512);
    L.ff1_b = A.f32(s.get(p + "ff1.ln.b"), 512);
    L.ff1_w1 = A.act(s.get(p + "ff1.w1"), 2048 * 512, bf);
    L.ff1_b1 = A.f32(s.get(p + "ff1.b1"), 2048);
    L.ff1_w2 = A.act(s.get(p + "ff1.w2"), 512 * 2048, bf);
    L.ff1_b2 = A.f32(s.get(p + "ff1.b2"), 512);
    L.att_g = A.f32(s.get(p + "att.ln.g"), 512);
    L.att_b = A.f32(s.get(p + "att.ln.b"), 512);
    {
      std::vector<float> w, b;
      if (have) {
        w.resize(1536 * 512);
        b.resize(1536);
        const char* nm[3] = {"q", "k", "v"};
        for (int i = 0; i < 3; ++i) {
          std::memcpy(&w[(size_t)i * 512 * 512], s.get(p + "att.w" + nm[i]), 512 * 512 * 4);
          std::memcpy(&b[(size_t)i * 512], s.get(p + "att.b" + nm[i]), 512 * 4);
        }
      }
      L.wqkv = A.act(have ? w.data() : nullptr, 1536 * 512, bf);
      L.bqkv = A.f32(have ? b.data() : nullptr, 1536);
    }
    L.wo = A.act(s.get(p + "att.wo"), 512 * 512, bf);
    L.wo_f = bf ? A.frag(s.get(p + "att.wo"), 512, 512) : nullptr;
    L.bo = A.f32(s.get(p + "att.bo"), 512);
    L.u = A.f32(s.get(p + "att.u"), 512);
    L.v = A.f32(s.get(p + "att.v"), 512);
    {  // positional projection, fp32 copy of the (possibly bf16-valued) matrix
      std::vector<float> w;
      if (have) {
        w.assign(s.get(p + "att.wpos"), s.get(p + "att.wpos") + 512 * 512);
        if (bf)
          for (auto& x : w) {
            uint32_t u;
            std::memcpy(&u, &x, 4);
            u += 0x7FFFu + ((u >> 16) & 1u);
            u &= 0xFFFF0000u;
            std::memcpy(&x, &u, 4);
          }
      }
      L.wpos = const_cast<float*>(A.f32(have ? w.data() : nullptr, 512 * 512));
    }
    L.P = A.raw((size_t)(2 * SF_MAX_WINDOW - 1) * 512 * m->esz);
    if (l == 0)  // split-K scratch of the projection GEMMs at init
      m->init_part = static_cast<float*>(A.raw((size_t)(2 * SF_MAX_WINDOW - 1) * 4 * 512 * 4));
    L.conv_g = A.f32(s.get(p + "conv.ln.g"), 512);
    L.conv_b = A.f32(s.get(p + "conv.ln.b"), 512);
    {  // pointwise-1 rows interleaved in blocks of 16 (value, gate) for the GLU epilogue
      std::vector<float> w, b;
      if (have) {
        w.resize(1024 * 512);
        b.resize(1024);
        const float* sw = s.get(p + "conv.pw1.w");
        const float* sb = s.get(p + "conv.pw1.b");
        for (int r = 0; r < 1024; ++r) {
          const int q = r / 32, i = r % 32;
          const int src = i < 16 ? 16 * q + i : 512 + 16 * q + (i - 16);
          std::memcpy(&w[(size_t)r * 512], sw + (size_t)src * 512, 512 * 4);
          b[r] = sb[src];
        }
      }
      L.pw1 = A.act(have ? w.data() : nullptr, 1024 * 512, bf);
      L.pw1_b = A.f32(have ? b.data() : nullptr, 1024);
    }
    L.dw9 = A.f32(s.get(p + "conv.dw.w"), 512 * 9);
    {  // BatchNorm (eval) and the depthwise bias folded into scale/shift
      std::vector<float> sc, sh;
      if (have) {
        sc.resize(512);
        sh.resize(512);
        const float *g = s.get(p + "conv.bn.g"), *bb = s.get(p + "conv.bn.b"),
                    *mu = s.get(p + "conv.bn.mean"), *var = s.get(p + "conv.bn.var"),
                    *db = s.get(p + "conv.dw.b");
        for (int c = 0; c < 512; ++c) {
          const double k = (double)g[c] / std::sqrt((double)var[c] + 1e-5);
          sc[c] = (float)k;
          sh[c] = (float)((double)bb[c] + k * ((double)db[c] - (double)mu[c]));
        }
      }
      L.dw_sc = A.f32(have ? sc.data() : nullptr, 512);
      L.dw_sh = A.f32(have ? sh.data() : nullptr, 512);
    }
    L.pw2 = A.act(s.get(p + "conv.pw2.w"), 512 * 512, bf);
    L.pw2_b = A.f32(s.get(p + "conv.pw2.b"), 512);
    L.ff2_g = A.f32(s.get(p + "ff2.ln.g"), 512);
    L.ff2_b = A.f32(s.get(p + "ff2.ln.b"), 512);
    L.ff2_w1 = A.act(s.get(p + "ff2.w1"), 2048 * 512, bf);
    L.ff2_b1 = A.f32(s.get(p + "ff2.b1"), 2048);
    L.ff2_w2 = A.act(s.get(p + "ff2.w2"), 512 * 2048, bf);
    L.ff2_b2 = A.f32(s.get(p + "ff2.b2"), 512);
    L.out_g = A.f32(s.get(p + "out_ln.g"), 512);
    L.out_b = A.f32(s.get(p + "out_ln.b"), 512);
  }
  m->proj_w = A.act(s.get("proj.w"), 192 * 512, bf);
  m->proj_b = A.f32(s.get("proj.b"), 192);
  for (int l = 0; l < 18; ++l) {
    const std::string p = "tf" + std::to_string(l) + ".";
    TfLayer& L = m->tf[l];
    std::vector<float> w, b;
    if (have) {
      w.resize(576 * 192);
      b.resize(576);
      const char* nm[3] = {"q", "k", "v"};
      for (int i = 0; i < 3; ++i) {
        std::memcpy(&w[(size_t)i * 192 * 192], s.get(p + "w" + nm[i]), 192 * 192 * 4);
        std::memcpy(&b[(size_t)i * 192], s.get(p + "b" + nm[i]), 192 * 4);
      }
    }
    L.wqkv = A.act(have ? w.data() : nullptr, 576 * 192, bf);
    L.bqkv = A.f32(have ? b.data() : nullptr, 576);
    L.wo = A.act(s.get(p + "wo"), 192 * 192, bf);
    L.bo = A.f32(s.get(p + "bo"), 192);
    L.ln1_g = A.f32(s.get(p + "ln1.g"), 192);
    L.ln1_b = A.f32(s.get(p + "ln1.b"), 192);
    L.w1 = A.act(s.get(p + "w1"), 768 * 192, bf);
    L.b1 = A.f32(s.get(p + "b1"), 768);
    L.w2 = A.act(s.get(p + "w2"), 192 * 768, bf);
    L.b2 = A.f32(s.get(p + "b2"), 192);
    L.ln2_g = A.f32(s.get(p + "ln2.g"), 192);
    L.ln2_b = A.f32(s.get(p + "ln2.b"), 192);
    if (bf) {  // operand copies for the fused layer tail
      L.wo_f = A.frag(s.get(p + "wo"), 192, 192);
      L.w1_f = A.frag(s.get(p + "w1"), 768, 192);
      L.w2_f = A.frag(s.get(p + "w2"), 192, 768);
      L.wqkv_f = A.frag(have ? w.data() : nullptr, 576, 192);
    }
  }
  {
    // fp32 MFMA fragment order: fragment (ks, ct) holds, for lane l,
    // W1[16ct + l%16][4ks + l/16]
    std::vector<float> w1f;
    if (have) {
      w1f.resize(192 * 192);
      const float* w = s.get("head.w1");
      for (int ks = 0; ks < 48; ++ks)
        for (int ct = 0; ct < 12; ++ct)
          for (int l = 0; l < 64; ++l)
            w1f[((size_t)ks * 12 + ct) * 64 + l] = w[(16 * ct + l % 16) * 192 + 4 * ks + l / 16];
    }
    m->h_w1f = A.f32(have ? w1f.data() : nullptr, 192 * 192);
    m->h_b1 = A.f32(s.get("head.b1"), 192);
    m->h_w2 = A.f32(s.get("head.w2"), (size_t)m->cfg.n_spk * 192);
    m->h_b2 = A.f32(s.get("head.b2"), m->cfg.n_spk);
  }
  {  // interleaved sinusoids for relative distances -(Wmax-1) .. Wmax-1
    std::vector<float> pe;
    if (have) {
      pe.resize((size_t)(2 * SF_MAX_WINDOW - 1) * 512);
      for (int r = 0; r < 2 * SF_MAX_WINDOW - 1; ++r) {
        const double delta = r - (SF_MAX_WINDOW - 1);
        for (int k = 0; k < 256; ++k) {
          const double om = std::pow(10000.0, -2.0 * k / 512.0);
          pe[(size_t)r * 512 + 2 * k] = (float)std::sin(delta * om);
          pe[(size_t)r * 512 + 2 * k + 1] = (float)std::cos(delta * om);
        }
      }
    }
    m->pe = const_cast<float*>(A.f32(have ? pe.data() : nullptr, (size_t)(2 * SF_MAX_WINDOW - 1) * 512));
  }
}

void build_nemotron(sf_model* m, Arena& A, const Src& s) {
  const bool bf = m->bf16;
  const bool have = s.w != nullptr;
  m->in_w = A.act(s.get("in.w"), 512 * 1024, bf);
  m->in_b = A.f32(s.get("in.b"), 512);
  for (int l = 0; l < 31; ++l) {
    const std::string p = "rl" + std::to_string(l) + ".";
    TfLayer& L = m->rl[l];
    L.ln1_g = A.f32(s.get(p + "ln1.g"), 512);
    L.ln1_b = A.f32(s.get(p + "ln1.b"), 512);
    std::vector<float> w, b;
    if (have) {
      w.resize(1536 * 512);
      b.resize(1536);
      const char* nm[3] = {"q", "k", "v"};
      for (int i = 0; i < 3; ++i) {
        std::memcpy(&w[(size_t)i * 512 * 512], s.get(p + "w" + nm[i]), 512 * 512 * 4);
        std::memcpy(&b[(size_t)i * 512], s.get(p + "b" + nm[i]), 512 * 4);
      }
    }
    L.wqkv = A.act(have ? w.data() : nullptr, 1536 * 512, bf);
    L.bqkv = A.f32(have ? b.data() : nullptr, 1536);
    L.wo = A.act(s.get(p + "wo"), 512 * 512, bf);
    L.wo_f = bf ? A.frag(s.get(p + "wo"), 512, 512) : nullptr;
    L.bo = A.f32(s.get(p + "bo"), 512);
    L.ln2_g = A.f32(s.get(p + "ln2.g"), 512);
    L.ln2_b = A.f32(s.get(p + "ln2.b"), 512);
    L.w1 = A.act(s.get(p + "w1"), 2048 * 512, bf);
    L.b1 = A.f32(s.get(p + "b1"), 2048);
    L.w2 = A.act(s.get(p + "w2"), 512 * 2048, bf);
    L.b2 = A.f32(s.get(p + "b2"), 512);
  }
  m->fin_g = A.f32(s.get("final_ln.g"), 512);
  m->fin_b = A.f32(s.get("final_ln.b"), 512);
  m->nh_w = A.f32(s.get("head.w"), 8 * 512);
  m->nh_b = A.f32(s.get("head.b"), 8);
  m->up_w = A.f32(s.get("up.w"), 8 * 8 * 8);
  m->up_b = A.f32(s.get("up.b"), 8);
  std::vector<float> rope;
  if (have) {  // rotate-half tables: angle = pos * 10000^(-i/32), i < 32
    rope.resize((size_t)SF_MAX_WINDOW * 64);
    for (int pos = 0; pos < SF_MAX_WINDOW; ++pos)
      for (int i = 0; i < 32; ++i) {
        const double ang = pos * std::pow(10000.0, -(double)i / 32.0);
        rope[((size_t)pos * 32 + i) * 2] = (float)std::cos(ang);
        rope[((size_t)pos * 32 + i) * 2 + 1] = (float)std::sin(ang);
      }
  }
  m->rope = A.f32(have ? rope.data() : nullptr, (size_t)SF_MAX_WINDOW * 64);
}

void build(sf_model* m, Arena& A, const Src& s) {
  if (m->cfg.arch == SF_ARCH_SORTFORMER) build_sortformer(m, A, s);
  else build_nemotron(m, A, s);
  std::vector<float> tab;
  if (s.w) tab = frontend_table();
  m->fe_tab = A.f32(s.w ? tab.data() : nullptr, 1680 + 128 * 32);
}
}  // namespace

bool valid_config(const sf_model_config* c) {
  if (!c) return false;
  if (c->arch != SF_ARCH_SORTFORMER && c->arch != SF_ARCH_NEMOTRON) return false;
  if (c->dtype != SF_DTYPE_F32 && c->dtype != SF_DTYPE_BF16) return false;
  if (c->init_mode != SF_INIT_SPEC && c->init_mode != SF_INIT_FULL_RANDOM) return false;
  if (c->arch == SF_ARCH_SORTFORMER && c->n_spk != 4) return false;
  if (c->arch == SF_ARCH_NEMOTRON && c->n_spk != 8) return false;
  return true;
}

size_t weight_bytes(const sf_model_config* c) {
  if (!valid_config(c)) return 0;
  sf_model tmp{};
  tmp.cfg = *c;
  tmp.bf16 = c->dtype == SF_DTYPE_BF16;
  tmp.esz = tmp.bf16 ? 2 : 4;
  tmp.list = c->arch == SF_ARCH_SORTFORMER ? sortformer_list(c->n_spk) : nemotron_list(c->n_spk);
  Arena A;
  build(&tmp, A, Src{&tmp.list, nullptr});
  return (A.off + 255) & ~(size_t)255;
}

sf_status init_model(sf_model* m, void* d_weights, size_t bytes, hipStream_t st) {
  m->bf16 = m->cfg.dtype == SF_DTYPE_BF16;
  m->esz = m->bf16 ? 2 : 4;
  m->list = m->cfg.arch == SF_ARCH_SORTFORMER ? sortformer_list(m->cfg.n_spk)
                                              : nemotron_list(m->cfg.n_spk);
  std::vector<std::vector<float>> w;
  generate(m->list, m->seed, m->cfg.init_mode == SF_INIT_FULL_RANDOM, w);
  const size_t need = weight_bytes(&m->cfg);
  if (bytes < need) return SF_ENOMEM;
  std::vector<char> host(need, 0);
  Arena A;
  A.dev = static_cast<char*>(d_weights);
  A.host = host.data();
  build(m, A, Src{&m->list, &w});
  m->base = static_cast<char*>(d_weights);
  m->bytes = need;
  if (hipMemcpyAsync(d_weights, host.data(), need, hipMemcpyHostToDevice, st) != hipSuccess)
    return SF_EHIP;
  if (m->cfg.arch == SF_ARCH_SORTFORMER) {
    // p(delta) = W_pos pe(delta) for every representable delta, per layer
    for (int l = 0; l < 17; ++l) {
      GemmArgs g{};
      g.A = m->pe; g.lda = 512;
      g.W = m->conf[l].wpos; g.ldw = 512;
      g.bias = nullptr;
      g.M = 2 * SF_MAX_WINDOW - 1; g.N = 512; g.K = 512;
      g.out = m->conf[l].P; g.ldo = 512;
      g.part = m->init_part; g.max_split = 4;
      gemm(g, EPI_STORE, false, m->bf16, st);
    }
  }
  if (take_gemm_failure()) return SF_ENOMEM;
  if (hipStreamSynchronize(st) != hipSuccess) return SF_EHIP;
  if (hipGetLastError() != hipSuccess) return SF_EHIP;
  return SF_OK;
}

// ---------------------------------------------------------- workspaces
// fp32 scratch for split-K partial sums of the encoder: room for
// [slices][rows][N] with slices * N <= 4096.
size_t part_floats(size_t rows) { return rows * 4096; }

size_t enc_ws_bytes(const sf_model* m, int B, int W) {
  const size_t r = (size_t)B * W, es = m->esz;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t t = 0;
  t += al(r * 512 * 4);   // x
  t += al(r * 512 * es);  // h
  t += al(r * 2048 * es); // big
  t += al(r * 512 * es);  // ctx
  t += al(r * 512 * 4);   // glu
  t += al(r * 8 * 4);     // probs
  t += al(r * 64 * 4);    // probs10
  t += al(part_floats(r) * 4);
  t += al((size_t)B * 512 * (W + 8) * es);  // V transposed per head
  t += 256;                                  // valid length of a fixed window
  return t;
}

EncWs carve_enc(const sf_model* m, char* p, int B, int W) {
  const size_t r = (size_t)B * W, es = m->esz;
  auto take = [&](size_t bytes) {
    char* q = p;
    p += (bytes + 255) & ~(size_t)255;
    return q;
  };
  EncWs w;
  w.x = reinterpret_cast<float*>(take(r * 512 * 4));
  w.h = take(r * 512 * es);
  w.big = take(r * 2048 * es);
  w.ctx = take(r * 512 * es);
  w.glu = reinterpret_cast<float*>(take(r * 512 * 4));
  w.probs = reinterpret_cast<float*>(take(r * 8 * 4));
  w.probs10 = reinterpret_cast<float*>(take(r * 64 * 4));
  w.part_floats = part_floats(r);
  w.part = reinterpret_cast<float*>(take(w.part_floats * 4));
  w.vpitch = (W + 7) / 8 * 8;
  w.vt = take((size_t)B * 512 * (W + 8) * es);
  w.nv = reinterpret_cast<int*>(take(256));
  return w;
}

size_t pre_ws_bytes(const sf_model* m, int B, int n) {
  const size_t es = m->esz, b = B, nn = n + 1;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t t = al(b * (8 * nn) * 128 * 4);  // mel
  if (m->cfg.arch == SF_ARCH_SORTFORMER) {
    t += al(b * (4 * nn) * 64 * 256 * 4);  // conv0 out
    t += al(b * (2 * nn) * 32 * 256 * es); // dw1 out
    t += al(b * (2 * nn) * 32 * 256 * 4);  // pw1 out
    t += al(b * nn * 16 * 256 * es);       // dw2 out
    t += al(b * nn * 16 * 256 * es);       // pw2 out
  } else {
    t += al(b * nn * 1024 * es);           // stacked frames
  }
  t += al(b * nn * PART_PER_ROW * 4);  // split-K partials
  return t;
}

// Encoder frames [e0, e1) of every stream from audio. Audio sample s of
// stream b is audio[b*a_bstride + (s & ring_mask)]; samples >= n_total are
// zero. T = mel frames of the utterance known so far. Output rows go to
// dst + b*dst_bstride + (j-e0)*512 (fp32).
void pre_encode_range(const sf_model* m, const float* audio, long long a_bstride,
                      long long ring_mask, long long n_total, int T, int e0, int e1, int B,
                      float* dst, long long dst_bstride, char* wsp, hipStream_t s) {
  const int n = e1 - e0;
  if (n <= 0) return;
  const bool bf = m->bf16;
  const size_t es = m->esz;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* p = wsp;
  const size_t nn = n + 1;
  float* mel = reinterpret_cast<float*>(p);
  p += al((size_t)B * 8 * nn * 128 * 4);
  if (m->cfg.arch == SF_ARCH_SORTFORMER) {
    const int T1 = (T + 1) / 2, T2 = (T1 + 1) / 2;
    const int t0 = std::max(0, 8 * e0 - 8), t1 = std::min(T, 8 * e1);
    const int a1 = std::max(0, 4 * e0 - 3), b1 = std::min(T1, 4 * e1);
    const int a2 = std::max(0, 2 * e0 - 1), b2 = std::min(T2, 2 * e1);
    float* part = reinterpret_cast<float*>(p);
    p += al((size_t)B * nn * PART_PER_ROW * 4);
    float* l1 = reinterpret_cast<float*>(p);
    p += al((size_t)B * 4 * nn * 64 * 256 * 4);
    void* d1 = p;
    p += al((size_t)B * 2 * nn * 32 * 256 * es);
    float* p1 = reinterpret_cast<float*>(p);
    p += al((size_t)B * 2 * nn * 32 * 256 * 4);
    void* d2 = p;
    p += al((size_t)B * nn * 16 * 256 * es);
    void* p2 = p;
    const long long mel_bs = (long long)(t1 - t0) * 128;
    logmel(audio, a_bstride, ring_mask, n_total, t0, t1 - t0, B, m->fe_tab, mel, mel_bs, s);
    const long long l1_bs = (long long)(b1 - a1) * 64 * 256;
    conv0(mel, mel_bs, t0, T, l1, l1_bs, a1, b1 - a1, B, m->c0_w, m->c0_b, s);
    const long long d1_bs = (long long)(b2 - a2) * 32 * 256;
    dw2d(l1, l1_bs, a1, T1, 64, d1, d1_bs, a2, b2 - a2, B, m->dw_w[0], m->dw_b[0], bf, s);
    GemmArgs g{};
    g.A = d1; g.lda = 256; g.W = m->pw_w[0]; g.ldw = 256; g.bias = m->pw_b[0];
    g.M = B * (b2 - a2) * 32; g.N = 256; g.K = 256; g.out = p1; g.ldo = 256;
    gemm(g, EPI_RELU, bf, false, s);
    const long long d2_bs = (long long)n * 16 * 256;
    dw2d(p1, d1_bs, a2, T2, 32, d2, d2_bs, e0, n, B, m->dw_w[1], m->dw_b[1], bf, s);
    g = GemmArgs{};
    g.A = d2; g.lda = 256; g.W = m->pw_w[1]; g.ldw = 256; g.bias = m->pw_b[1];
    g.M = B * n * 16; g.N = 256; g.K = 256; g.out = p2; g.ldo = 256;
    gemm(g, EPI_RELU, bf, bf, s);
    g = GemmArgs{};
    g.A = p2; g.lda = 4096; g.W = m->pre_out_w; g.ldw = 4096; g.bias = m->pre_out_b;
    g.M = B * n; g.N = 512; g.K = 4096; g.out = dst; g.ldo = 512; g.rpb = n; g.bstride = dst_bstride;
    g.part = part; g.max_split = PART_PER_ROW / 512;
    gemm(g, EPI_STORE, bf, false, s);
  } else {
    const int t0 = 8 * e0, t1 = std::min(T, 8 * e1);
    float* part = reinterpret_cast<float*>(p);
    p += al((size_t)B * nn * PART_PER_ROW * 4);
    void* st = p;
    const long long mel_bs = (long long)std::max(0, t1 - t0) * 128;
    logmel(audio, a_bstride, ring_mask, n_total, t0, t1 - t0, B, m->fe_tab, mel, mel_bs, s);
    stack8(mel, mel_bs, t0, T, e0, n, B, st, bf, s);
    GemmArgs g{};
    g.A = st; g.lda = 1024; g.W = m->in_w; g.ldw = 1024; g.bias = m->in_b;
    g.M = B * n; g.N = 512; g.K = 1024; g.out = dst; g.ldo = 512; g.rpb = n; g.bstride = dst_bstride;
    g.part = part; g.max_split = PART_PER_ROW / 512;
    gemm(g, EPI_STORE, bf, false, s);
  }
}

// ------------------------------------------------------------- encoders
namespace {
struct Ctx {
  const sf_model* m;
  EncWs& w;
  int M;
  hipStream_t s;
  bool bf;
  // Linear with a fused epilogue into `out`.
  void lin(const void* A, int lda, const void* W, const float* bias, int N, int K, void* out,
           int ldo, int epi, bool bf_out, float* resid = nullptr, int ldr = 0) {
    GemmArgs g{};
    g.A = A; g.lda = lda; g.W = W; g.ldw = K; g.bias = bias; g.M = M; g.N = N; g.K = K;
    g.out = out; g.ldo = ldo; g.resid = resid; g.ldr = ldr;
    g.part = w.part; g.max_split = (int)(w.part_floats / ((size_t)M * N));
    gemm(g, epi, bf, bf_out, s);
  }
  // Fused Q/K/V projection: Q and K into `out`, V transposed per head into w.vt.
  void qkv(const void* A, int d, const void* W, const float* bias, void* out, int hd, int rows) {
    GemmArgs g{};
    g.A = A; g.lda = d; g.W = W; g.ldw = d; g.bias = bias; g.M = M; g.N = 3 * d; g.K = d;
    g.out = out; g.ldo = 3 * d;
    g.part = w.part; g.max_split = (int)(w.part_floats / ((size_t)M * 3 * d));
    g.vt = w.vt; g.vcol = 2 * d; g.vrows = rows; g.vpitch = w.vpitch; g.vhd = hd;
    gemm(g, EPI_QKV, bf, bf, s);
  }
  // Residual-branch Linear: fp32 partial sums for the next LayerNorm.
  int branch(const void* A, int lda, const void* W, int N, int K) {
    GemmArgs g{};
    g.A = A; g.lda = lda; g.W = W; g.ldw = K; g.M = M; g.N = N; g.K = K;
    g.out = w.part; g.ldo = N; g.max_split = (int)(w.part_floats / ((size_t)M * N));
    return gemm(g, EPI_PARTIAL, bf, false, s);
  }
  // x += alpha * (A W^T + bias) (N = 512), then the LayerNorm(s) as in ln():
  // batched bf16 windows add the branch in the GEMM's epilogue (x_mode 1,
  // storing the updated residual, is then already done); otherwise the GEMM
  // writes partial slices that the LayerNorm sums and adds
  void branch_ln(const void* A, int lda, const void* W, int K, const float* bias, float alpha,
                 const float* g1, const float* b1, const float* g2, const float* b2, int x_mode,
                 void* y) {
    if (bf && M > SLICE_MAX_ROWS) {
      GemmArgs g{};
      g.A = A; g.lda = lda; g.W = W; g.ldw = K; g.M = M; g.N = 512; g.K = K; g.bias = bias;
      g.out = w.x; g.ldo = 512; g.ralpha = alpha;
      if (gemm_resid(g, s) == 1) {
        ln(512, 0, nullptr, 0.f, g1, b1, g2, b2, x_mode == 1 ? 0 : x_mode, y);
        return;
      }
    }
    const int ns = branch(A, lda, W, 512, K);
    ln(512, ns, bias, alpha, g1, b1, g2, b2, x_mode, y);
  }
  // LayerNorm(s) with the pending residual branch (ns partial slices) folded in.
  void ln(int D, int ns, const float* pbias, float alpha, const float* g1, const float* b1,
          const float* g2, const float* b2, int x_mode, void* y_act) {
    LnArgs a{};
    a.x = w.x; a.M = M; a.D = D;
    a.part = ns > 0 ? w.part : nullptr; a.nsplit = ns; a.pbias = pbias; a.alpha = alpha;
    a.g1 = g1; a.b1 = b1; a.g2 = g2; a.b2 = b2; a.x_mode = x_mode; a.y_act = y_act;
    layernorm(a, bf, s);
  }
};
}  // namespace

namespace {
// Copies of registered (layer, point) activations, widened to fp32.
struct Taps {
  const sf_model* m;
  bool on;
  long long rows;
  hipStream_t s;
  void at(int layer, int point, const void* src, bool src_bf16, int d) const {
    if (!on) return;
    for (const auto& t : m->taps)
      if (t.layer == layer && t.point == point) widen(src, src_bf16, t.out, rows * d, s);
  }
};
}  // namespace

int tap_layers(const sf_model* m) { return m->cfg.arch == SF_ARCH_SORTFORMER ? 35 : 31; }
int tap_width(const sf_model* m, int layer) {
  return m->cfg.arch == SF_ARCH_SORTFORMER && layer >= 17 ? 192 : 512;
}

static void encode_sortformer(const sf_model* m, EncWs& w, int B, int W, int n_valid,
                              hipStream_t s, const Taps& tp, const int* nv) {
  const bool bf = m->bf16;
  Ctx c{m, w, B * W, s, bf};
  c.ln(512, 0, nullptr, 0.f, m->conf[0].ff1_g, m->conf[0].ff1_b, nullptr, nullptr, 0, w.h);
  for (int l = 0; l < 17; ++l) {
    const ConfLayer& L = m->conf[l];
    tp.at(l, SF_TAP_LAYER_IN, w.x, false, 512);
    // macaron FFN, first half: x += FF(LN(x))/2
    c.lin(w.h, 512, L.ff1_w1, L.ff1_b1, 2048, 512, w.big, 2048, EPI_SWISH, bf);
    c.branch_ln(w.big, 2048, L.ff1_w2, 2048, L.ff1_b2, 0.5f, L.att_g, L.att_b, nullptr, nullptr, 1,
                w.h);
    // relative-position self-attention
    c.qkv(w.h, 512, L.wqkv, L.bqkv, w.big, 64, W);
    AttnArgs a{};
    a.qkv = w.big; a.ldq = 1536; a.qoff = 0; a.koff = 512; a.vt = w.vt; a.vpitch = w.vpitch;
    a.B = B; a.H = 8; a.W = W; a.n_valid = n_valid; a.nv = nv;
    a.ub = L.u; a.vb = L.v; a.P = L.P; a.ldp = 512; a.p_center = SF_MAX_WINDOW - 1;
    a.ctx = w.ctx; a.ldc = 512; a.scale = 0.125f;
    // windows in the latency form: the output projection's per-head partial
    // sums come from the attention kernel itself
    const bool fuse_wo = bf && B * W <= SLICE_MAX_ROWS;
    if (fuse_wo) { a.wo_f = L.wo_f; a.part = w.part; a.M = B * W; }
    attention(a, ATT_RELPOS, 64, bf, s);
    tp.at(l, SF_TAP_ATTN_CTX, w.ctx, bf, 512);
    if (fuse_wo) c.ln(512, 8, L.bo, 1.f, L.conv_g, L.conv_b, nullptr, nullptr, 1, w.h);
    else c.branch_ln(w.ctx, 512, L.wo, 512, L.bo, 1.f, L.conv_g, L.conv_b, nullptr, nullptr, 1, w.h);
    // convolution module
    if (bf && B * W <= SLICE_MAX_ROWS) {
      // pointwise-1, GLU, depthwise conv, BatchNorm and Swish in one kernel
      // (into ctx: h is its input)
      GemmArgs g{};
      g.A = w.h; g.lda = 512; g.W = L.pw1; g.ldw = 512; g.bias = L.pw1_b;
      g.M = B * W; g.N = 1024; g.K = 512; g.out = w.ctx; g.ldo = 512;
      g.dw_w9 = L.dw9; g.dw_sc = L.dw_sc; g.dw_sh = L.dw_sh; g.dw_W = W; g.dw_nvalid = n_valid;
      g.dw_nv = nv;
      gemm_glu_dwconv(g, s);
      c.branch_ln(w.ctx, 512, L.pw2, 512, L.pw2_b, 1.f, L.ff2_g, L.ff2_b, nullptr, nullptr, 1, w.h);
    } else {
      // (batched bf16 windows: the GLU output goes to the depthwise conv as bf16)
      c.lin(w.h, 512, L.pw1, L.pw1_b, 1024, 512, w.glu, 512, EPI_GLU, bf);
      dwconv_time(w.glu, bf, B, W, n_valid, nv, L.dw9, L.dw_sc, L.dw_sh, w.h, bf, s);
      c.branch_ln(w.h, 512, L.pw2, 512, L.pw2_b, 1.f, L.ff2_g, L.ff2_b, nullptr, nullptr, 1, w.h);
    }
    // macaron FFN, second half, then the output LayerNorm (fused with the
    // next layer's first LayerNorm)
    c.lin(w.h, 512, L.ff2_w1, L.ff2_b1, 2048, 512, w.big, 2048, EPI_SWISH, bf);
    if (l < 16) {
      c.branch_ln(w.big, 2048, L.ff2_w2, 2048, L.ff2_b2, 0.5f, L.out_g, L.out_b,
                  m->conf[l + 1].ff1_g, m->conf[l + 1].ff1_b, 2, w.h);
      tp.at(l, SF_TAP_LAYER_OUT, w.x, false, 512);
    } else {
      c.branch_ln(w.big, 2048, L.ff2_w2, 2048, L.ff2_b2, 0.5f, L.out_g, L.out_b, nullptr, nullptr,
                  0, w.h);
      tp.at(l, SF_TAP_LAYER_OUT, w.h, bf, 512);
    }
  }
  // encoder_proj: fp32 residual stream of the transformer + GEMM operand
  c.lin(w.h, 512, m->proj_w, m->proj_b, 192, 512, w.ctx, 192, EPI_STORE, bf, w.x, 192);
  const void* hin = w.ctx;
  // batched bf16 windows: each layer's tail kernel also projects the next
  // layer's Q/K/V, so only the first layer runs the Q/K/V GEMM
  const bool tail_qkv = bf && B * W > SLICE_MAX_ROWS;
  for (int l = 0; l < 18; ++l) {
    const TfLayer& L = m->tf[l];
    tp.at(17 + l, SF_TAP_LAYER_IN, w.x, false, 192);
    if (!tail_qkv || l == 0) c.qkv(hin, 192, L.wqkv, L.bqkv, w.big, 24, W);
    AttnArgs a{};
    a.qkv = w.big; a.ldq = 576; a.qoff = 0; a.koff = 192; a.vt = w.vt; a.vpitch = w.vpitch;
    a.B = B; a.H = 8; a.W = W; a.n_valid = n_valid; a.nv = nv;
    a.ctx = w.ctx; a.ldc = 192; a.scale = 1.0f / std::sqrt(24.0f);
    attention(a, ATT_PLAIN, 24, bf, s);
    tp.at(17 + l, SF_TAP_ATTN_CTX, w.ctx, bf, 192);
    if (bf && !tail_qkv) {
      // output projection, LN1 and the FFN's two Linears in one kernel (x1 kept
      // in the fp32 GLU buffer, which the transformer does not otherwise use)
      TfTailArgs t{};
      t.ctx = w.ctx; t.x = w.x; t.x1 = w.glu; t.M = B * W;
      t.wo = L.wo_f; t.bo = L.bo; t.g1 = L.ln1_g; t.be1 = L.ln1_b;
      t.w1 = L.w1_f; t.b1 = L.b1; t.w2 = L.w2_f; t.part = w.part;
      const int nc = tf_tail(t, s);
      LnArgs n{};
      n.x = w.x; n.x_in = w.glu; n.M = B * W; n.D = 192;
      n.part = w.part; n.nsplit = nc; n.pbias = L.b2; n.alpha = 1.f;
      n.g1 = L.ln2_g; n.b1 = L.ln2_b; n.x_mode = 2; n.y_act = w.h;
      layernorm(n, bf, s);
    } else if (tail_qkv) {
      // batched windows: the whole tail in one kernel
      TfLayerArgs t{};
      t.ctx = w.ctx; t.x = w.x; t.xo = w.x; t.h = w.h; t.M = B * W;
      t.wo = L.wo_f; t.bo = L.bo; t.g1 = L.ln1_g; t.be1 = L.ln1_b;
      t.w1 = L.w1_f; t.b1 = L.b1; t.w2 = L.w2_f; t.b2 = L.b2; t.g2 = L.ln2_g; t.be2 = L.ln2_b;
      if (l < 17) {  // the next layer's Q/K/V from the same kernel; h is not needed then
        const TfLayer& N = m->tf[l + 1];
        t.h = nullptr;
        t.wqkv = N.wqkv_f; t.bqkv = N.bqkv; t.qkv = w.big; t.vt = w.vt;
        t.vrows = W; t.vpitch = w.vpitch;
      }
      tf_layer_tp(t, s);
    } else {
      int ns = c.branch(w.ctx, 192, L.wo, 192, 192);
      c.ln(192, ns, L.bo, 1.f, L.ln1_g, L.ln1_b, nullptr, nullptr, 2, w.h);   // post-LN
      c.lin(w.h, 192, L.w1, L.b1, 768, 192, w.big, 768, EPI_RELU, bf);
      ns = c.branch(w.big, 768, L.w2, 192, 768);
      c.ln(192, ns, L.b2, 1.f, L.ln2_g, L.ln2_b, nullptr, nullptr, 2, w.h);
    }
    tp.at(17 + l, SF_TAP_LAYER_OUT, w.x, false, 192);
    hin = w.h;
  }
  head_sortformer(w.x, B * W, m->h_w1f, m->h_b1, m->h_w2, m->h_b2, m->cfg.n_spk, w.probs, s);
}

static void encode_nemotron(const sf_model* m, EncWs& w, int B, int W, int n_valid,
                            hipStream_t s, const Taps& tp, const int* nv) {
  const bool bf = m->bf16;
  Ctx c{m, w, B * W, s, bf};
  c.ln(512, 0, nullptr, 0.f, m->rl[0].ln1_g, m->rl[0].ln1_b, nullptr, nullptr, 0, w.h);
  for (int l = 0; l < 31; ++l) {
    const TfLayer& L = m->rl[l];
    tp.at(l, SF_TAP_LAYER_IN, w.x, false, 512);
    c.qkv(w.h, 512, L.wqkv, L.bqkv, w.big, 64, W);
    AttnArgs a{};
    a.qkv = w.big; a.ldq = 1536; a.qoff = 0; a.koff = 512; a.vt = w.vt; a.vpitch = w.vpitch;
    a.B = B; a.H = 8; a.W = W; a.n_valid = n_valid; a.nv = nv; a.rope = m->rope;
    a.ctx = w.ctx; a.ldc = 512; a.scale = 0.125f;
    const bool fuse_wo = bf && B * W <= SLICE_MAX_ROWS;  // as in the conformer layers
    if (fuse_wo) { a.wo_f = L.wo_f; a.part = w.part; a.M = B * W; }
    attention(a, ATT_ROPE, 64, bf, s);
    tp.at(l, SF_TAP_ATTN_CTX, w.ctx, bf, 512);
    // pre-LN
    if (fuse_wo) c.ln(512, 8, L.bo, 1.f, L.ln2_g, L.ln2_b, nullptr, nullptr, 1, w.h);
    else c.branch_ln(w.ctx, 512, L.wo, 512, L.bo, 1.f, L.ln2_g, L.ln2_b, nullptr, nullptr, 1, w.h);
    c.lin(w.h, 512, L.w1, L.b1, 2048, 512, w.big, 2048, EPI_GELU, bf);
    if (l < 30)
      c.branch_ln(w.big, 2048, L.w2, 2048, L.b2, 1.f, m->rl[l + 1].ln1_g, m->rl[l + 1].ln1_b,
                  nullptr, nullptr, 1, w.h);
    else  // final LN, into x
      c.branch_ln(w.big, 2048, L.w2, 2048, L.b2, 1.f, m->fin_g, m->fin_b, nullptr, nullptr, 2,
                  nullptr);
    tp.at(l, SF_TAP_LAYER_OUT, w.x, false, 512);
  }
  head_nemotron(w.x, B * W, m->nh_w, m->nh_b, m->up_w, m->up_b, w.probs, w.probs10, s);
}

void encode(const sf_model* m, EncWs& w, int B, int W, int n_valid, hipStream_t s, bool taps,
            const int* nv) {
  const Taps tp{m, taps && !m->taps.empty(), (long long)B * W, s};
  if (m->cfg.arch == SF_ARCH_SORTFORMER) encode_sortformer(m, w, B, W, n_valid, s, tp, nv);
  else encode_nemotron(m, w, B, W, n_valid, s, tp, nv);
}

}  // namespace sfm
