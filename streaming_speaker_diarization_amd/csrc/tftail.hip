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
