// Host-side structures of the library: tensor lists, the device weight
// arena of a model, and the streaming state.
#pragma once
#include <cstdint>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "sortformer.h"

namespace sfh {

struct TSpec {
  std::string name;
  std::vector<int64_t> shape;
  char kind;  // 'w' random, 'b' zero/bias, 'g' one/gain
  int64_t numel() const {
    int64_t n = 1;
    for (auto d : shape) n *= d;
    return n;
  }
};

std::vector<TSpec> sortformer_list(int n_spk);
std::vector<TSpec> nemotron_list(int n_spk);
void generate(const std::vector<TSpec>& list, uint64_t seed, bool full_random,
              std::vector<std::vector<float>>& out);

// Device pointers of one conformer layer.
struct ConfLayer {
  const float *ff1_g, *ff1_b, *att_g, *att_b, *conv_g, *conv_b, *ff2_g, *ff2_b, *out_g, *out_b;
  const void *ff1_w1, *ff1_w2, *wqkv, *wo, *pw1, *pw2, *ff2_w1, *ff2_w2;
  const float *ff1_b1, *ff1_b2, *bqkv, *bo, *pw1_b, *pw2_b, *ff2_b1, *ff2_b2;
  const float *u, *v, *dw9, *dw_sc, *dw_sh;
  const void* wo_f;  // bf16 fragment-major copy of wo (output projection fused into attention)
  float* wpos;  // fp32 positional projection (init only)
  void* P;      // (2*SF_MAX_WINDOW-1, 512) projected relative positions
};
struct TfLayer {
  const void *wqkv, *wo, *w1, *w2;
  const void *wo_f, *w1_f, *w2_f;  // bf16 fragment-major copies (fused layer tail)
  const void* wqkv_f;               // bf16 fragment-major Q/K/V (batched layer tail)
  const float *bqkv, *bo, *b1, *b2, *ln1_g, *ln1_b, *ln2_g, *ln2_b;
};

}  // namespace sfh

struct sf_model {
  struct Tap {
    int layer, point;
    float* out;
    size_t cap;  // floats
  };
  sf_model_config cfg;
  bool bf16;
  size_t esz;  // bytes per GEMM operand element
  uint64_t seed;
  char* base;
  size_t bytes;
  std::vector<sfh::TSpec> list;
  // Sortformer
  const float *c0_w, *c0_b, *dw_w[2], *dw_b[2], *pw_b[2], *pre_out_b;
  const void *pw_w[2], *pre_out_w;
  sfh::ConfLayer conf[17];
  const void* proj_w;
  const float* proj_b;
  sfh::TfLayer tf[18];
  const float *h_w1f, *h_b1, *h_w2, *h_b2;
  float* pe;
  float* init_part;  // split-K scratch used while deriving the position tables
  // Nemotron
  const void* in_w;
  const float* in_b;
  sfh::TfLayer rl[31];
  const float *fin_g, *fin_b, *nh_w, *nh_b, *up_w, *up_b, *rope;
  // frontend tables
  const float* fe_tab;
  // NEMOTRON output frames: 10 ms x out_stride (1, 2, 4 or 8)
  int out_stride;
  // per-layer taps honoured by sortformer_encode_window
  std::vector<Tap> taps;
};

struct sf_stream {
  sf_model* m;
  sf_stream_config sc;
  int B, S, D;
  int cap;             // rows of the [cache | FIFO | look-ahead] buffer
  long long ring_cap;  // audio ring samples (power of two)
  float* E[2];
  float* P[2];
  int* ph[2];
  int cur;
  double* sil_sum;
  int* sil_cnt;
  int* slots;  // compression slot map (B, cap)
  float* ring;
  int Lc, Lf, Lp;
  long long steps, emitted, recv;
  long long pending;  // samples fed past recv, held in the ring for the next step
  int enc_done;
  bool finished;
  bool rows_only;     // rows written by sortformer_stream_set_rows: steps refused until
                      // a reset or a checkpoint import makes the counters consistent
  // window-forward graphs keyed by (window rows, ping-pong buffer, workspace)
  // (HIP handles kept opaque here: this header is also built by the host compiler)
  bool use_graphs;
  bool fixed_window;  // every window padded to cap rows, one graph per ping-pong buffer
  void* cap_stream;                                            // hipStream_t
  std::map<std::tuple<int, int, const void*>, void*> graphs;   // hipGraphExec_t
  const void* graph_ws;  // the workspace the cached graphs were captured with
};
