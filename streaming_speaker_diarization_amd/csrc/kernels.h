// Launch interfaces of the gfx950 kernels. Every launcher only enqueues on
// the given stream; shapes are validated by the host code that calls them.
#pragma once
#include <hip/hip_ext.h>

#include "common.h"
#include "sortformer.h"

namespace sf {

enum { EPI_STORE = 0, EPI_SWISH = 1, EPI_RELU = 2, EPI_GELU = 3, EPI_GLU = 5, EPI_PARTIAL = 6,
       EPI_QKV = 7, EPI_RESID = 8 };
// Windows up to this many rows use the K-slice GEMM kernel.
#define SLICE_MAX_ROWS 4096
// fp32 partial-sum scratch per GEMM row: slices * N never exceeds this
// (bf16: 4 x 512 residual branches; fp32: 8 x 512 or 2 x 2048; the 4096->512
// subsampling output: 8 x 512 bf16, 16 x 512 fp32).
#define PART_PER_ROW 8192

struct GemmArgs {
  const void* A; int lda;   // (M, K) activations
  const void* W; int ldw;   // (N, K) weights
  const float* bias;        // (N) or null
  int M, N, K;
  void* out; int ldo;       // (M, N) output (EPI_GLU: (M, N/2))
  int rpb;                  // rows per batch of the output (0: contiguous)
  long long bstride;        // output elements between batches when rpb != 0
  float* resid; int ldr;    // EPI_STORE: optional fp32 copy of the output
  void* part;               // fp32 scratch for split-K partial sums (may be null)
  int max_split;            // most K slices the scratch (or, for EPI_PARTIAL, out) holds
  // EPI_QKV: columns >= vcol (the V block) go to vt transposed per head,
  // vt[((b*H + h)*hd + d)*vpitch + w] for row m = b*vrows + w.
  void* vt; int vcol, vrows, vpitch, vhd;
  // gemm_glu_dwconv only: depthwise conv (k = 9) weights [512][9], folded
  // BatchNorm scale / shift, and the stream layout of the rows (m = b*dw_W +
  // frame; frames at or past dw_nvalid count as zero).
  const float* dw_w9; const float* dw_sc; const float* dw_sh;
  int dw_W, dw_nvalid;
  const int* dw_nv;  // when non-null: device copy of the valid frame count, read instead
  float ralpha;      // gemm_resid: out (fp32) += ralpha * (A W^T + bias)
};
// EPI_PARTIAL writes fp32 partial sums (no bias) to out as [slice][M][N] and
// returns the slice count; other epilogues return 1.
int gemm(const GemmArgs& g, int epi, bool bf16_in, bool bf16_out, hipStream_t s);
// Residual branch of batched windows (bf16 A and W, more than 4096 rows,
// K % 64 == 0, N % 64 == 0): out (fp32, ldo) += ralpha * (A W^T + bias), in
// place, with the arithmetic of a LayerNorm that folds in one partial slice.
// Returns 1, or -1 (nothing launched) for other shapes.
int gemm_resid(const GemmArgs& g, hipStream_t s);
// Pointwise-1 of the conformer convolution module (bf16, N = 1024 GLU
// interleaved, K = 512) with the GLU, the depthwise conv (k = 9), the folded
// BatchNorm and the Swish fused into its epilogue: out (M, 512) bf16. Each
// workgroup computes 4 halo rows on either side of its 24 output rows, so the
// convolution needs nothing from other workgroups. Windows of up to 4096 rows;
// returns 1, or -1 (nothing launched) for other shapes.
int gemm_glu_dwconv(const GemmArgs& g, hipStream_t s);
// True (and cleared) if a gemm() call since the last check launched nothing
// because its partial-sum scratch was missing or too small.
bool take_gemm_failure();
// Records that a launcher refused its arguments (reported by take_gemm_failure).
void flag_launch_failure();

enum { ATT_PLAIN = 0, ATT_RELPOS = 1, ATT_ROPE = 2 };
struct AttnArgs {
  const void* qkv; int ldq;   // (B*W, ldq) rows, q/k column blocks
  int qoff, koff;
  const void* vt; int vpitch; // V transposed per head: (B, H, hd, vpitch), keys contiguous
  int B, H, W, n_valid;
  const int* nv;      // when non-null: device copy of n_valid, read instead (fixed windows)
  const float* ub; const float* vb;   // (H, hd) relative-position biases
  const void* P; int ldp; int p_center; // relative-position projections, row delta+p_center
  const float* rope;                  // (max_window, hd/2) (cos, sin) pairs
  void* ctx; int ldc;                 // (B*W, ldc) output
  float scale;
  // Optional (bf16 latency form, ATT_RELPOS / ATT_ROPE, H*hd == 512): the output
  // projection's partial sums per head, part[h][M][512] = ctx_h Wo[:, h]^T
  // (M = B*W rows, no bias), with wo_f the fragment-major Wo (Arena::frag).
  const void* wo_f; float* part; int M;
};
void attention(const AttnArgs& a, int mode, int head_dim, bool bf16, hipStream_t s);

// LayerNorm over rows of the fp32 residual stream x (D = 512 or 192), with
// the residual branch folded in: v = x + alpha*(sum_s part[s] + pbias) when
// part is given (split-K partials of the branch's last Linear, [s][M][D]).
// x_mode: 0 leave x, 1 x <- v, 2 x <- LN1(v). y_act <- LN2(LN1(v)) if g2
// else LN1(v) (GEMM operand type), when non-null.
struct LnArgs {
  float* x; int M; int D;
  const float* x_in;  // residual read from here instead of x when non-null
  const float* part; int nsplit; const float* pbias; float alpha;
  const float *g1, *b1, *g2, *b2;
  int x_mode;
  void* y_act;
};
void layernorm(const LnArgs& a, bool bf16, hipStream_t s);

// Post-LN transformer layer tail (d = 192, FFN 768), bf16, up to 4096 rows:
// x1 = LN1(x + ctx Wo^T + bo) written to x1 (fp32), and the FFN's output
// projection as fp32 partial sums over hidden chunks, part[c][M][192] (bias
// b2 not included), for a LayerNorm with x_in = x1. wo, w1, w2 are in
// fragment-major order (Arena::frag). Returns the number of chunks.
#ifndef SF_TFT_NCH
#define SF_TFT_NCH 4
#define SF_TFT_NW 4
#endif
struct TfTailArgs {
  const void* ctx; const float* x; float* x1; int M;
  const void* wo; const float* bo; const float* g1; const float* be1;
  const void* w1; const float* b1; const void* w2;
  float* part;
};
int tf_tail(const TfTailArgs& a, hipStream_t s);

// The same layer tail for batched windows (more than 4096 rows), with the FFN
// output projection and LN2 in the kernel as well:
//   x1 = LN1(x + ctx Wo^T + bo); xo = LN2(x1 + relu(x1 W1^T + b1) W2^T + b2)
// and h = bf16(xo), the next layer's GEMM operand. xo may alias x (each
// workgroup reads its rows before writing them). wo, w1, w2 fragment-major.
// With wqkv (fragment-major [576][192]) the next layer's Q/K/V projection of
// xo follows in the same kernel: Q and K row-major into qkv (576 columns), V
// transposed per head into vt[((b*8 + head)*24 + d)*vpitch + w] for row
// m = b*vrows + w; h may then be null (not written).
struct TfLayerArgs {
  const void* ctx; const float* x; float* xo; void* h; int M;
  const void* wo; const float* bo; const float* g1; const float* be1;
  const void* w1; const float* b1; const void* w2; const float* b2;
  const float* g2; const float* be2;
  const void* wqkv; const float* bqkv; void* qkv; void* vt; int vrows, vpitch;
};
void tf_layer_tp(const TfLayerArgs& a, hipStream_t s);

// nv (may be null): device copy of n_valid, read instead when given. glu is
// (B*W, 512), fp32 or (glu_bf16, with a bf16 output only) bf16.
void dwconv_time(const void* glu, bool glu_bf16, int B, int W, int n_valid, const int* nv,
                 const float* w9, const float* scale, const float* shift, void* out, bool bf16,
                 hipStream_t s);

void logmel(const float* audio, long long a_bstride, long long ring_mask, long long n_total,
            long long t0, int nfr, int B, const float* tables, float* mel, long long m_bstride,
            hipStream_t s);

void conv0(const float* mel, long long mel_bstride, int mel_base, int T, float* out,
           long long out_bstride, int o_base, int n_out, int B, const float* w, const float* b,
           hipStream_t s);
void dw2d(const float* in, long long in_bstride, int in_base, int len_in, int f_in, void* out,
          long long out_bstride, int o_base, int n_out, int B, const float* w, const float* b,
          bool bf16, hipStream_t s);
void stack8(const float* mel, long long mel_bstride, int mel_base, int T, int e0, int n, int B,
            void* out, bool bf16, hipStream_t s);

void head_sortformer(const float* x, int M, const float* w1f, const float* b1, const float* w2,
                     const float* b2, int S, float* probs, hipStream_t s);
void head_nemotron(const float* x, int M, const float* hw, const float* hb, const float* uw,
                   const float* ub, float* p80, float* p10, hipStream_t s);

void copy_rows(const float* src, long long s_bstride, int s_ld, float* dst, long long d_bstride,
               int d_ld, int B, int rows, int cols, hipStream_t s);
// dst[b][k][c] = mean of src[b][r k + q][c] over q < r (rows of S = cols
// floats, dense): n_out output rows per batch
void pool_rows(const float* src, long long s_bstride, float* dst, long long d_bstride, int B,
               int n_out, int r, int cols, hipStream_t s);
// copy_rows for `rows` rows per batch where rows at or past the device count
// *nv are written as zeros
void copy_rows_nv(const float* src, long long s_bstride, int s_ld, float* dst, long long d_bstride,
                  int d_ld, int B, int rows, int cols, const int* nv, hipStream_t s);
// n contiguous elements (fp32, or bf16 when src_bf16) widened to fp32
void widen(const void* src, bool src_bf16, float* dst, long long n, hipStream_t s);
// n samples of each stream (stream b's at src + b*src_bstride) into the audio
// ring at absolute positions start .. start+n-1 (modulo the power-of-two cap)
void ring_write(const float* src, long long src_bstride, long long n_new, int B, float* ring,
                long long ring_cap, long long start, hipStream_t s);
void fill_i32(int* p, long long n, int v, hipStream_t s);
void fill_f64(double* p, long long n, double v, hipStream_t s);
void refresh_probs(const float* win_probs, int W, int S, int B, int Lc, int nrows, float* P,
                   int* ph, int cap, hipStream_t s);
void silence_update(const float* E, const float* P, int cap, int D, int S, int B, int r0, int n,
                    double* sil_sum, int* sil_cnt, hipStream_t s);
void compress_cache(const float* E, const float* P, const int* ph, int cap, int D, int S, int B,
                    int M, int tail, const double* sil_sum, const int* sil_cnt, int C, int per,
                    int k, float* E2, float* P2, int* ph2, int* slots, hipStream_t s);

// Probabilities (B, T, S) -> per-track segments (see segments.hip).
void segments(const float* probs, int B, int T, int S, double dt, const sf_segment_params& prm,
              sf_segment* out, long long cap, long long* counts, hipStream_t s);

// Benchmark profiling (see prof.hip). Classes match SF_PROF_* in the ABI.
enum { PROF_GEMM = 1, PROF_ATTN = 2, PROF_LN = 3, PROF_CONV = 4, PROF_FRONTEND = 5, PROF_CACHE = 6 };
bool prof_active(int cls);
// Next event pair of the pool (and the launch's algorithmic flops/bytes).
void prof_next(hipEvent_t* start, hipEvent_t* stop, double flops, double bytes);
int prof_start(int cls, int max_launches);
int prof_stop(double* ms, long long* launches, double* flops, double* bytes);
bool profiling();  // any class being profiled (graph capture is then bypassed)

// Launches a kernel; while its class is profiled the launch carries a start
// and a stop event recorded by the dispatch itself, so the timed interval is
// exactly the kernel's execution.
// Arguments are converted to the kernel's parameter types before packing.
template <typename... KArgs, typename... Args>
inline void klaunch(int cls, double flops, double bytes, void (*kern)(KArgs...), dim3 grid,
                    dim3 block, hipStream_t s, Args... args) {
  if (prof_active(cls)) {
    hipEvent_t e0, e1;
    prof_next(&e0, &e1, flops, bytes);
    hipExtLaunchKernelGGL(kern, grid, block, 0, s, e0, e1, 0, static_cast<KArgs>(args)...);
  } else {
    hipLaunchKernelGGL(kern, grid, block, 0, s, static_cast<KArgs>(args)...);
  }
}

}  // namespace sf
