// Tail of a post-LN transformer layer (d = 192, FFN 768; model card,
// Pipeline: Transformer encoder) for windows of up to 4096 rows, bf16:
//   x1      = LN1(x + ctx Wo^T + bo)
//   part[c] = relu(x1 W1[c]^T + b1[c]) W2[:, c]^T   for hidden chunk c of 4
// in one kernel: one workgroup = 16 rows x one 192-wide hidden chunk, so every
// step is row-local (the output projection and LN1 are recomputed by the four
// chunk workgroups of a row block). The LayerNorm kernel that follows forms
// LN2(x1 + sum_c part[c] + b2). Weight fragments are read straight from
// global memory into registers (each is used by one wave only); the LN1
// output and the hidden activations pass through LDS to become MFMA A
// operands.
#include "kernels.h"

namespace sf {

namespace {
constexpr int TD = 192, TF = 768, THC = 4, TFC = TF / THC, TNK = TD / 32, TLH = TD + 8;
}

__global__ __launch_bounds__(256) void tf_tail_kernel(TfTailArgs a) {
  using M_ = MF<bf16_t>;
  __shared__ __align__(16) bf16_t hs[16 * TLH];  // LN1 output (bf16)
  __shared__ __align__(16) bf16_t hc[16 * TLH];  // relu(x1 W1[c]^T + b1[c]) (bf16)
  __shared__ float red[4][16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int chunk = blockIdx.x, r0 = blockIdx.y * 16;
  const bf16_t* ctx = static_cast<const bf16_t*>(a.ctx);
  const bf16_t* Wo = static_cast<const bf16_t*>(a.wo);
  const bf16_t* W1 = static_cast<const bf16_t*>(a.w1);
  const bf16_t* W2 = static_cast<const bf16_t*>(a.w2);

  // ---- loads: ctx rows (A), Wo rows 48w.. (B), the chunk's W1 rows (B, step 3)
  bf16x8_t af[TNK], bw[3][TNK], b1f[3][TNK];
  {
    const int r = min(r0 + c16, a.M - 1);
#pragma unroll
    for (int ks = 0; ks < TNK; ++ks)
      af[ks] = *reinterpret_cast<const bf16x8_t*>(ctx + (size_t)r * TD + ks * 32 + 8 * g);
  }
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int ks = 0; ks < TNK; ++ks) {
      const int n = 48 * w + 16 * j + c16;
      bw[j][ks] = *reinterpret_cast<const bf16x8_t*>(Wo + (size_t)n * TD + ks * 32 + 8 * g);
      b1f[j][ks] = *reinterpret_cast<const bf16x8_t*>(W1 + (size_t)(chunk * TFC + n) * TD +
                                                      ks * 32 + 8 * g);
    }
  // ---- y = ctx Wo^T
  f32x4 acc[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < TNK; ++ks)
#pragma unroll
    for (int j = 0; j < 3; ++j) acc[j] = M_::mma(af[ks], bw[j][ks], acc[j]);
  // the chunk's W2 columns for step 4 (reusing the Wo registers)
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int ks = 0; ks < TNK; ++ks)
      bw[j][ks] = *reinterpret_cast<const bf16x8_t*>(W2 + (size_t)(48 * w + 16 * j + c16) * TF +
                                                     chunk * TFC + ks * 32 + 8 * g);

  // ---- x1 = LN1(x + y + bo): lane holds rows 4g+r, columns 48w+16j+c16
  float v[3][4];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int col = 48 * w + 16 * j + c16;
    const float bo = a.bo[col];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = min(r0 + 4 * g + r, a.M - 1);
      v[j][r] = a.x[(size_t)row * TD + col] + (acc[j][r] + bo);
    }
  }
  float mean[4], rstd[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float s = row16_sum(v[0][r] + v[1][r] + v[2][r]);
    if (c16 == 0) red[w][4 * g + r] = s;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r)
    mean[r] = (red[0][4 * g + r] + red[1][4 * g + r] + red[2][4 * g + r] + red[3][4 * g + r]) *
              (1.0f / TD);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      v[j][r] -= mean[r];
      q += v[j][r] * v[j][r];
    }
    q = row16_sum(q);
    if (c16 == 0) red[w][4 * g + r] = q;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r)
    rstd[r] = 1.0f / sqrtf((red[0][4 * g + r] + red[1][4 * g + r] + red[2][4 * g + r] +
                            red[3][4 * g + r]) * (1.0f / TD) + 1e-5f);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int col = 48 * w + 16 * j + c16;
    const float gg = a.g1[col], bb = a.be1[col];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x1 = v[j][r] * rstd[r] * gg + bb;
      const int row = r0 + 4 * g + r;
      if (chunk == 0 && row < a.M) a.x1[(size_t)row * TD + col] = x1;
      hs[(4 * g + r) * TLH + col] = f2bf(x1);
    }
  }
  __syncthreads();

  // ---- hidden chunk: relu(x1 W1[c]^T + b1[c])
#pragma unroll
  for (int ks = 0; ks < TNK; ++ks) af[ks] = M_::ld(&hs[c16 * TLH + ks * 32], lane);
#pragma unroll
  for (int j = 0; j < 3; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < TNK; ++ks)
#pragma unroll
    for (int j = 0; j < 3; ++j) acc[j] = M_::mma(af[ks], b1f[j][ks], acc[j]);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int col = 48 * w + 16 * j + c16;
    const float bb = a.b1[chunk * TFC + col];
#pragma unroll
    for (int r = 0; r < 4; ++r) hc[(4 * g + r) * TLH + col] = f2bf(fmaxf(acc[j][r] + bb, 0.f));
  }
  __syncthreads();

  // ---- partial of the output projection over this hidden chunk
#pragma unroll
  for (int ks = 0; ks < TNK; ++ks) af[ks] = M_::ld(&hc[c16 * TLH + ks * 32], lane);
#pragma unroll
  for (int j = 0; j < 3; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < TNK; ++ks)
#pragma unroll
    for (int j = 0; j < 3; ++j) acc[j] = M_::mma(af[ks], bw[j][ks], acc[j]);
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = r0 + 4 * g + r;
      if (row < a.M)
        a.part[((size_t)chunk * a.M + row) * TD + 48 * w + 16 * j + c16] = acc[j][r];
    }
}

int tf_tail(const TfTailArgs& a, hipStream_t s) {
  if (a.M <= 0) return THC;
  const double M = a.M;
  klaunch(PROF_GEMM, 2.0 * M * TD * TD + 4.0 * M * TD * TF,
          2.0 * M * TD + 4.0 * M * TD * 2 + 2.0 * (TD * TD + 2.0 * TD * TF) + 4.0 * THC * M * TD,
          tf_tail_kernel, dim3(THC, (a.M + 15) / 16), dim3(256), s, a);
  return THC;
}

}  // namespace sf
