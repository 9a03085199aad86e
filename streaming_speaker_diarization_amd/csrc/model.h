// Internal interface between the C ABI and the forward graphs.
#pragma once
#include <hip/hip_runtime.h>

#include "host.h"

namespace sfm {

struct EncWs {
  float* x;       // (B*W, 512) fp32 residual stream (192 columns in the transformer)
  void* h;        // (B*W, 512) GEMM operand
  void* big;      // (B*W, 2048) FFN hidden / fused QKV
  void* ctx;      // (B*W, 512) attention output
  float* glu;     // (B*W, 512) GLU output
  float* probs;   // (B*W, S) 80 ms probabilities
  float* probs10; // (B*8W, S) 10 ms probabilities (Nemotron)
  float* part;    // split-K partial sums of residual-branch Linears
  size_t part_floats;
  void* vt;       // (B, H, head dim, vpitch) V transposed per head
  int vpitch;     // keys per V^T row (window rounded up to 8)
  int* nv;        // one int: the valid window length of a fixed padded window
};

bool valid_config(const sf_model_config* c);
size_t weight_bytes(const sf_model_config* c);
sf_status init_model(sf_model* m, void* d_weights, size_t bytes, hipStream_t st);
size_t enc_ws_bytes(const sf_model* m, int B, int W);
EncWs carve_enc(const sf_model* m, char* p, int B, int W);
size_t pre_ws_bytes(const sf_model* m, int B, int n);
void pre_encode_range(const sf_model* m, const float* audio, long long a_bstride,
                      long long ring_mask, long long n_total, int T, int e0, int e1, int B,
                      float* dst, long long dst_bstride, char* wsp, hipStream_t s);
// taps: honour m->taps (the caller has checked their capacities)
// nv (may be null): device copy of n_valid, which the kernels then read instead
// (windows of a fixed padded size whose valid length changes per replay)
void encode(const sf_model* m, EncWs& w, int B, int W, int n_valid, hipStream_t s,
            bool taps = false, const int* nv = nullptr);
int tap_layers(const sf_model* m);
int tap_width(const sf_model* m, int layer);

}  // namespace sfm
