// Tail of a post-LN transformer layer (d = 192, FFN 768; model card,
// Pipeline: Transformer encoder) for windows of up to 4096 rows, bf16:
//   x1      = LN1(x + ctx Wo^T + bo)
//   part[c] = relu(x1 W1[c]^T + b1[c]) W2[:, c]^T   for hidden chunk c
// in one kernel: one workgroup = 16 rows x one hidden chunk, so every step is
// row-local (the output projection and LN1 are recomputed by the chunk
// workgroups of a row block). The LayerNorm kernel that follows forms
// LN2(x1 + sum_c part[c] + b2). The weights come in fragment-major order
// (one 1 KB block per 16 x 32 MFMA operand, lane l's 16 bytes at 16 l), so
// each wave's weight loads read whole cache lines; every load of the
// workgroup is issued before the first product. The LN1 output and the
// hidden activations pass through LDS to become MFMA A operands.
#include "kernels.h"

namespace sf {

namespace {
constexpr int TD = 192, TF = 768, TLH = TD + 8;
}

// NCH hidden chunks, NW waves: wave w owns output columns CW*w.. and hidden
// columns HC/NW*w.. of its chunk
template <int NCH, int NW>
__global__ __launch_bounds__(NW * 64) void tf_tail_kernel(TfTailArgs a) {
  using M_ = MF<bf16_t>;
  constexpr int HC = TF / NCH;         // hidden columns per chunk
  constexpr int CW = TD / NW;          // output columns per wave
  constexpr int OT = CW / 16;          // output tiles per wave
  constexpr int HT = HC / 16 / NW;     // hidden tiles per wave
  constexpr int NK = TD / 32;          // k-steps over d
  constexpr int NKH = HC / 32;         // k-steps over the chunk's hidden columns
  constexpr int TLC = HC + 8;
  static_assert(CW % 16 == 0 && HC % (16 * NW) == 0 && HC % 32 == 0, "tail tiling");
  __shared__ __align__(16) bf16_t hs[16 * TLH];  // LN1 output (bf16)
  __shared__ __align__(16) bf16_t hc[16 * TLC];  // hidden activations (bf16)
  __shared__ float red[NW][16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int chunk = blockIdx.x, r0 = blockIdx.y * 16;
  const bf16_t* ctx = static_cast<const bf16_t*>(a.ctx);
  // fragment (tile t, k-step s) of a matrix with K columns: block t*(K/32)+s
  auto frag = [&](const void* m, int K, int t, int s) {
    return *reinterpret_cast<const bf16x8_t*>(static_cast<const bf16_t*>(m) +
                                              ((size_t)t * (K / 32) + s) * 512 + 8 * lane);
  };

  bf16x8_t af[NK], bw[OT][NK], b1f[HT][NK], b2f[OT][NKH];
  {
    const int r = min(r0 + c16, a.M - 1);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      af[ks] = *reinterpret_cast<const bf16x8_t*>(ctx + (size_t)r * TD + ks * 32 + 8 * g);
  }
#pragma unroll
  for (int j = 0; j < OT; ++j)
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) bw[j][ks] = frag(a.wo, TD, OT * w + j, ks);
#pragma unroll
  for (int j = 0; j < HT; ++j)
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) b1f[j][ks] = frag(a.w1, TD, chunk * (HC / 16) + HT * w + j, ks);
#pragma unroll
  for (int j = 0; j < OT; ++j)
#pragma unroll
    for (int ks = 0; ks < NKH; ++ks) b2f[j][ks] = frag(a.w2, TF, OT * w + j, chunk * NKH + ks);
  float xr[OT][4], bo[OT], g1[OT], be1[OT], b1v[HT];
#pragma unroll
  for (int j = 0; j < OT; ++j) {
    const int col = CW * w + 16 * j + c16;
    bo[j] = a.bo[col];
    g1[j] = a.g1[col];
    be1[j] = a.be1[col];
#pragma unroll
    for (int r = 0; r < 4; ++r) xr[j][r] = a.x[(size_t)min(r0 + 4 * g + r, a.M - 1) * TD + col];
  }
#pragma unroll
  for (int j = 0; j < HT; ++j) b1v[j] = a.b1[chunk * HC + (HT * w + j) * 16 + c16];

  // ---- y = ctx Wo^T
  f32x4 acc[OT > HT ? OT : HT];
#pragma unroll
  for (int j = 0; j < OT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NK; ++ks)
#pragma unroll
    for (int j = 0; j < OT; ++j) acc[j] = M_::mma(af[ks], bw[j][ks], acc[j]);

  // ---- x1 = LN1(x + y + bo): lane holds rows 4g+r, columns CW*w+16j+c16
  float v[OT][4];
#pragma unroll
  for (int j = 0; j < OT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) v[j][r] = xr[j][r] + (acc[j][r] + bo[j]);
  float mean[4], rstd[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < OT; ++j) s += v[j][r];
    s = row16_sum(s);
    if (c16 == 0) red[w][4 * g + r] = s;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < NW; ++u) s += red[u][4 * g + r];
    mean[r] = s * (1.0f / TD);
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < OT; ++j) {
      v[j][r] -= mean[r];
      q += v[j][r] * v[j][r];
    }
    q = row16_sum(q);
    if (c16 == 0) red[w][4 * g + r] = q;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float q = 0.f;
#pragma unroll
    for (int u = 0; u < NW; ++u) q += red[u][4 * g + r];
    rstd[r] = 1.0f / sqrtf(q * (1.0f / TD) + 1e-5f);
  }
#pragma unroll
  for (int j = 0; j < OT; ++j) {
    const int col = CW * w + 16 * j + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x1 = v[j][r] * rstd[r] * g1[j] + be1[j];
      const int row = r0 + 4 * g + r;
      if (chunk == 0 && row < a.M) a.x1[(size_t)row * TD + col] = x1;
      hs[(4 * g + r) * TLH + col] = f2bf(x1);
    }
  }
  __syncthreads();

  // ---- this wave's hidden columns of the chunk: relu(x1 W1[c]^T + b1[c])
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) af[ks] = M_::ld(&hs[c16 * TLH + ks * 32], lane);
#pragma unroll
  for (int j = 0; j < HT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NK; ++ks)
#pragma unroll
    for (int j = 0; j < HT; ++j) acc[j] = M_::mma(af[ks], b1f[j][ks], acc[j]);
#pragma unroll
  for (int j = 0; j < HT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      hc[(4 * g + r) * TLC + (HT * w + j) * 16 + c16] = f2bf(fmaxf(acc[j][r] + b1v[j], 0.f));
  __syncthreads();

  // ---- partial of the output projection over this hidden chunk
  bf16x8_t ah[NKH];
#pragma unroll
  for (int ks = 0; ks < NKH; ++ks) ah[ks] = M_::ld(&hc[c16 * TLC + ks * 32], lane);
#pragma unroll
  for (int j = 0; j < OT; ++j) {
    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKH; ++ks) acc[j] = M_::mma(ah[ks], b2f[j][ks], acc[j]);
  }
#pragma unroll
  for (int j = 0; j < OT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = r0 + 4 * g + r;
      if (row < a.M)
        a.part[((size_t)chunk * a.M + row) * TD + CW * w + 16 * j + c16] = acc[j][r];
    }
}

// ---------------------------------------------------------------------------
// Throughput form (batched windows, more than 4096 rows): the whole layer tail
//   x1 = LN1(x + ctx Wo^T + bo),  x <- LN2(x1 + relu(x1 W1^T + b1) W2^T + b2)
// in one kernel, h <- x as the next GEMM operand (bf16). One workgroup = 48
// rows (each wave's chain of products is the kernel's limit, so the rows go
// to as many workgroups as two per CU allow); wave w owns output columns
// 48w .. 48w+47 of every 192-wide product (3 tiles x 3 row tiles, so each
// weight fragment it loads feeds 3 products) and, in each of the 4 hidden
// chunks of 192, hidden columns 48w .. 48w+47.
// The A operands (ctx, then x1, and each hidden chunk) sit in LDS as bf16 for
// all four waves; row statistics of both LayerNorms are reduced across the
// waves through LDS. The output projection of the hidden layer accumulates
// over the chunks in registers, so no partial sums leave the kernel.
namespace {
constexpr int TB_RB = 48, TB_NW = 4, TB_CT = 3, TB_RT = TB_RB / 16, TB_NK = TD / 32;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void tf_layer_tp_kernel(TfLayerArgs a) {
  using M_ = MF<bf16_t>;
  __shared__ __align__(16) bf16_t As[TB_RB * TLH];  // ctx rows, then x1 (bf16)
  __shared__ __align__(16) bf16_t Hs[TB_RB * TLH];  // one hidden chunk (bf16)
  __shared__ float red[TB_NW][TB_RB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int r0 = blockIdx.x * TB_RB;
  auto frag = [&](const void* m, int K, int t, int s) {
    return *reinterpret_cast<const bf16x8_t*>(static_cast<const bf16_t*>(m) +
                                              ((size_t)t * (K / 32) + s) * 512 + 8 * lane);
  };
  // ---- ctx rows into LDS (16-byte chunks, rows past M clamped)
  {
    const bf16_t* ctx = static_cast<const bf16_t*>(a.ctx);
    constexpr int CPR = TD / 8;  // 24 chunks per row
#pragma unroll
    for (int i = 0; i < (TB_RB * CPR + 255) / 256; ++i) {
      const int c = tid + 256 * i, r = c / CPR, q = c % CPR;
      if (c >= TB_RB * CPR) break;
      const int row = min(r0 + r, a.M - 1);
      *reinterpret_cast<vec16*>(&As[r * TLH + 8 * q]) =
          *reinterpret_cast<const vec16*>(ctx + (size_t)row * TD + 8 * q);
    }
  }
  // lane (g, c16) of wave w holds, for row tile rt and column tile ct, rows
  // r0 + 16rt + 4g + r (r < 4) of column 48w + 16ct + c16
  float xv[TB_RT][TB_CT][4];
#pragma unroll
  for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < TB_CT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        xv[rt][ct][r] = a.x[(size_t)min(r0 + 16 * rt + 4 * g + r, a.M - 1) * TD + 48 * w + 16 * ct + c16];
  __syncthreads();

  f32x4 acc[TB_RT][TB_CT];
  auto zero = [&]() {
#pragma unroll
    for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < TB_CT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // acc += (rows of src) x M^T over K = 192 for this wave's 3 column tiles t0 + ct
  // (the product's 18 weight fragments are all requested before its first
  // MFMA, so it waits for the L2 once instead of once per k-step)
  auto product = [&](const bf16_t* src, const void* m, int K, int t0, int s0) {
    bf16x8_t bw[TB_NK][TB_CT];
#pragma unroll
    for (int ks = 0; ks < TB_NK; ++ks)
#pragma unroll
      for (int ct = 0; ct < TB_CT; ++ct) bw[ks][ct] = frag(m, K, t0 + ct, s0 + ks);
#pragma unroll
    for (int ks = 0; ks < TB_NK; ++ks) {
      bf16x8_t af[TB_RT];
#pragma unroll
      for (int rt = 0; rt < TB_RT; ++rt) af[rt] = M_::ld(&src[(16 * rt + c16) * TLH + ks * 32], lane);
#pragma unroll
      for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < TB_CT; ++ct) acc[rt][ct] = M_::mma(af[rt], bw[ks][ct], acc[rt][ct]);
    }
  };
  // LayerNorm over the 192 columns of every row of v (in place), gamma/beta
  // per column; the row sums are combined across the waves through LDS
  auto layernorm = [&](float (&v)[TB_RT][TB_CT][4], const float* gm, const float* bt) {
    float mean[TB_RT][4], rstd[TB_RT][4];
#pragma unroll
    for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float s = 0.f;
#pragma unroll
        for (int ct = 0; ct < TB_CT; ++ct) s += v[rt][ct][r];
        s = row16_sum(s);
        if (c16 == 0) red[w][16 * rt + 4 * g + r] = s;
      }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rt + 4 * g + r;
        mean[rt][r] = ((red[0][row] + red[1][row]) + (red[2][row] + red[3][row])) * (1.0f / TD);
      }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float q = 0.f;
#pragma unroll
        for (int ct = 0; ct < TB_CT; ++ct) {
          v[rt][ct][r] -= mean[rt][r];
          q += v[rt][ct][r] * v[rt][ct][r];
        }
        q = row16_sum(q);
        if (c16 == 0) red[w][16 * rt + 4 * g + r] = q;
      }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rt + 4 * g + r;
        rstd[rt][r] = 1.0f / sqrtf(((red[0][row] + red[1][row]) + (red[2][row] + red[3][row])) *
                                       (1.0f / TD) + 1e-5f);
      }
#pragma unroll
    for (int ct = 0; ct < TB_CT; ++ct) {
      const int col = 48 * w + 16 * ct + c16;
      const float gg = gm[col], bb = bt[col];
#pragma unroll
      for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[rt][ct][r] = v[rt][ct][r] * rstd[rt][r] * gg + bb;
    }
  };

  // ---- x1 = LN1(x + ctx Wo^T + bo)
  zero();
  product(As, a.wo, TD, 3 * w, 0);
#pragma unroll
  for (int ct = 0; ct < TB_CT; ++ct) {
    const float bo = a.bo[48 * w + 16 * ct + c16];
#pragma unroll
    for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) xv[rt][ct][r] = xv[rt][ct][r] + (acc[rt][ct][r] + bo);
  }
  layernorm(xv, a.g1, a.be1);  // its barriers also end every wave's reads of ctx
#pragma unroll
  for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < TB_CT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        As[(16 * rt + 4 * g + r) * TLH + 48 * w + 16 * ct + c16] = f2bf(xv[rt][ct][r]);
  __syncthreads();

  // ---- y = relu(x1 W1^T + b1) W2^T over 4 hidden chunks of 192
  f32x4 out[TB_RT][TB_CT];
#pragma unroll
  for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < TB_CT; ++ct) out[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < TF / TD; ++c) {
    zero();
    product(As, a.w1, TD, c * (TD / 16) + 3 * w, 0);
#pragma unroll
    for (int ct = 0; ct < TB_CT; ++ct) {
      const float b1 = a.b1[c * TD + 48 * w + 16 * ct + c16];
#pragma unroll
      for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Hs[(16 * rt + 4 * g + r) * TLH + 48 * w + 16 * ct + c16] =
              f2bf(fmaxf(acc[rt][ct][r] + b1, 0.f));
    }
    bf16x8_t bw[TB_NK][TB_CT];  // requested before the barrier, in flight while it waits
#pragma unroll
    for (int ks = 0; ks < TB_NK; ++ks)
#pragma unroll
      for (int ct = 0; ct < TB_CT; ++ct) bw[ks][ct] = frag(a.w2, TF, 3 * w + ct, c * TB_NK + ks);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < TB_NK; ++ks) {
      bf16x8_t ah[TB_RT];
#pragma unroll
      for (int rt = 0; rt < TB_RT; ++rt) ah[rt] = M_::ld(&Hs[(16 * rt + c16) * TLH + ks * 32], lane);
#pragma unroll
      for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < TB_CT; ++ct) out[rt][ct] = M_::mma(ah[rt], bw[ks][ct], out[rt][ct]);
    }
    __syncthreads();  // the next chunk rewrites Hs
  }

  // ---- x <- LN2(x1 + y + b2), h <- bf16(x)
#pragma unroll
  for (int ct = 0; ct < TB_CT; ++ct) {
    const float b2 = a.b2[48 * w + 16 * ct + c16];
#pragma unroll
    for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) xv[rt][ct][r] = xv[rt][ct][r] + (out[rt][ct][r] + b2);
  }
  layernorm(xv, a.g2, a.be2);
  bf16_t* h = static_cast<bf16_t*>(a.h);
  int gq = g;  // opaque copy: row indices recomputed, not kept from the x loads
  asm volatile("" : "+v"(gq));
#pragma unroll
  for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = r0 + 16 * rt + 4 * gq + r;
      if (row >= a.M) continue;
#pragma unroll
      for (int ct = 0; ct < TB_CT; ++ct) {
        const int col = 48 * w + 16 * ct + c16;
        const bf16_t hv = f2bf(xv[rt][ct][r]);
        a.xo[(size_t)row * TD + col] = xv[rt][ct][r];
        if (h) h[(size_t)row * TD + col] = hv;
        // the next layer's Q/K/V operand (As is free: the chunk loop ended
        // with a barrier after its last read)
        As[(16 * rt + 4 * g + r) * TLH + col] = hv;
      }
    }
  if (!a.wqkv) return;

  // ---- the next layer's Q/K/V projection of xo: pass p = 0, 1, 2 forms the
  // 192 columns of Q, K, V (wave w: column tiles 3w .. 3w+2 of the pass),
  // stages them in Hs as bf16 and stores them with 16-byte writes: Q and K
  // row-major (576 per row), V transposed per head (head dim 24, window rows
  // along the pitch). Rows of As past M hold finite values of a clamped row;
  // their outputs are not stored.
  __syncthreads();
  // an opaque copy of the thread index: the store indexing below is then
  // recomputed here rather than kept live (and spilled) from the ctx loads
  int tq = tid;
  asm volatile("" : "+v"(tq));
  bf16_t* qkv = static_cast<bf16_t*>(a.qkv);
  bf16_t* vt = static_cast<bf16_t*>(a.vt);
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    zero();
    product(As, a.wqkv, TD, 12 * pass + 3 * w, 0);
#pragma unroll
    for (int ct = 0; ct < TB_CT; ++ct) {
      const int col = 48 * w + 16 * ct + c16;
      const float bq = a.bqkv[TD * pass + col];
#pragma unroll
      for (int rt = 0; rt < TB_RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Hs[(16 * rt + 4 * g + r) * TLH + col] = f2bf(acc[rt][ct][r] + bq);
    }
    __syncthreads();
    if (pass < 2) {
      constexpr int CPR = TD / 8;
#pragma unroll
      for (int i = 0; i < (TB_RB * CPR + 255) / 256; ++i) {
        const int c = tq + 256 * i, r = c / CPR, q = c % CPR, row = r0 + r;
        if (c < TB_RB * CPR && row < a.M)
          *reinterpret_cast<vec16*>(qkv + (size_t)row * (3 * TD) + TD * pass + 8 * q) =
              *reinterpret_cast<const vec16*>(&Hs[r * TLH + 8 * q]);
      }
    } else if (a.vrows >= TB_RB) {
      // V^T: the block's rows fall in at most two windows, A and A+1; keys
      // go out in groups of 8 aligned to the window's own key index (whole
      // groups as 16-byte vectors, groups cut by the block edge or the
      // window's end element by element). A wave: 16 columns x 4 groups.
      const int W = a.vrows, m1 = min(r0 + TB_RB, a.M);
      const int bA = r0 / W, loA = r0 - bA * W, hiA = min(m1 - bA * W, W);
      const int gA0 = loA >> 3, nA = ((hiA - 1) >> 3) - gA0 + 1;
      const int hiB = m1 - (bA + 1) * W;
      const int nG = nA + (hiB > 0 ? ((hiB - 1) >> 3) + 1 : 0);
      constexpr int NG = (TB_RB / 8 + 2 + 3) / 4 * 4;
#pragma unroll 1
      for (int qi = tq; qi < TD * NG; qi += 256) {
        const int col = (qi / 64) % (TD / 16) * 16 + (qi & 15);
        const int gi = (qi / 64) / (TD / 16) * 4 + ((qi >> 4) & 3);
        if (gi >= nG) continue;
        const bool inA = gi < nA;
        const int bb = inA ? bA : bA + 1, grp = inA ? gA0 + gi : gi - nA;
        const int lo = inA ? loA : 0, hi = inA ? hiA : hiB;
        const int w0 = grp * 8, ws = max(w0, lo), we = min(w0 + 8, hi);
        const int rb = bb * W - r0;  // block row of key 0 of window bb
        const int hh = col / 24, d = col % 24;
        bf16_t* dst = vt + ((size_t)(bb * 8 + hh) * 24 + d) * a.vpitch + w0;
        if (ws == w0 && we == w0 + 8 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
          vec16 v;
          bf16_t* pv = reinterpret_cast<bf16_t*>(&v);
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = Hs[(rb + w0 + e) * TLH + col];
          *reinterpret_cast<vec16*>(dst) = v;
        } else {
          for (int w = ws; w < we; ++w) dst[w - w0] = Hs[(rb + w) * TLH + col];
        }
      }
    } else {
      // windows shorter than the block: 8-row runs of one V column
#pragma unroll 1
      for (int c = tq; c < TD * (TB_RB / 8); c += 256) {
        const int col = c / (TB_RB / 8), r = c % (TB_RB / 8) * 8, row = r0 + r;
        if (row >= a.M) continue;
        const int hh = col / 24, d = col % 24;
        for (int e = 0; e < 8 && row + e < a.M; ++e) {
          const int b2 = (row + e) / a.vrows, w2 = (row + e) % a.vrows;
          vt[((size_t)(b2 * 8 + hh) * 24 + d) * a.vpitch + w2] = Hs[(r + e) * TLH + col];
        }
      }
    }
    __syncthreads();  // the next pass rewrites Hs
  }
}

void tf_layer_tp(const TfLayerArgs& a, hipStream_t s) {
  if (a.M <= 0) return;
  const double M = a.M;
  const bool q = a.wqkv != nullptr;
  klaunch(PROF_GEMM, 2.0 * M * TD * TD + 4.0 * M * TD * TF + (q ? 2.0 * M * TD * 3 * TD : 0.0),
          2.0 * M * TD + 4.0 * M * TD * 2 + 2.0 * (TD * TD + 2.0 * TD * TF) +
              (q ? 2.0 * M * 3 * TD + 2.0 * 3 * TD * TD : 2.0 * M * TD),
          tf_layer_tp_kernel, dim3((a.M + TB_RB - 1) / TB_RB), dim3(256), s, a);
}

int tf_tail(const TfTailArgs& a, hipStream_t s) {
  constexpr int NCH = SF_TFT_NCH, NW = SF_TFT_NW;
  if (a.M <= 0) return NCH;
  const double M = a.M;
  klaunch(PROF_GEMM, 2.0 * M * TD * TD + 4.0 * M * TD * TF,
          2.0 * M * TD + 4.0 * M * TD * 2 + 2.0 * (TD * TD + 2.0 * TD * TF) + 4.0 * NCH * M * TD,
          tf_tail_kernel<NCH, NW>, dim3(NCH, (a.M + 15) / 16), dim3(NW * 64), s, a);
  return NCH;
}

}  // namespace sf
