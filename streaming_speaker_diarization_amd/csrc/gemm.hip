// Dense GEMM for every Linear layer of the forward: C[M,N] = A[M,K] * W[N,K]^T
// (PyTorch Linear layout, both operands K-contiguous) on MFMA, with the
// elementwise work that follows each Linear fused into the epilogue (bias,
// Swish, ReLU, GELU, GLU, scaled residual add).
//
// Tiling: 256 threads = 4 waves in a 2x2 grid; each wave owns a (BM/2)x(BN/2)
// sub-tile made of 16x16 MFMA tiles. A and W tiles of BK columns are staged
// through LDS (row stride padded by 16 bytes) with register double buffering:
// the next K tile is fetched from global memory while the current one feeds
// the matrix cores, and one barrier per K tile separates the two LDS buffers.
#include "kernels.h"

namespace sf {

template <typename T, typename OutT, int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int BK = sizeof(T) == 2 ? 64 : 32;
  constexpr int LDK = BK + VEC;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int CPR = BK / VEC;              // 16-byte chunks per tile row
  constexpr int A_IT = BM * CPR / 256;
  constexpr int B_IT = BN * CPR / 256;
  using M_ = MF<T>;
  __shared__ __align__(16) T As[2][BM * LDK];
  __shared__ __align__(16) T Bs[2][BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const T* A = static_cast<const T*>(g.A);
  const T* Wt = static_cast<const T*>(g.W);

  vec16 ra[A_IT], rb[B_IT];
  auto fetch = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      int c = tid + i * 256, r = c / CPR, kc = (c % CPR) * VEC;
      int m = m0 + r;
      if (m < g.M) ra[i] = *reinterpret_cast<const vec16*>(A + (size_t)m * g.lda + k0 + kc);
      else ra[i] = vec16{{0u, 0u, 0u, 0u}};
    }
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      int c = tid + i * 256, r = c / CPR, kc = (c % CPR) * VEC;
      rb[i] = *reinterpret_cast<const vec16*>(Wt + (size_t)(n0 + r) * g.ldw + k0 + kc);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      int c = tid + i * 256, r = c / CPR, kc = (c % CPR) * VEC;
      *reinterpret_cast<vec16*>(&As[buf][r * LDK + kc]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      int c = tid + i * 256, r = c / CPR, kc = (c % CPR) * VEC;
      *reinterpret_cast<vec16*>(&Bs[buf][r * LDK + kc]) = rb[i];
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = g.K / BK;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) fetch(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / M_::KI; ++ks) {
      typename M_::frag af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = M_::ld(&As[cur][(wm * WM + 16 * i + (lane & 15)) * LDK + ks * M_::KI], lane);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = M_::ld(&Bs[cur][(wn * WN + 16 * j + (lane & 15)) * LDK + ks * M_::KI], lane);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = M_::mma(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) stash(cur ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  OutT* out = static_cast<OutT*>(g.out);
  auto orow = [&](int m) -> size_t {
    return g.rpb ? (size_t)(m / g.rpb) * g.bstride + (size_t)(m % g.rpb) * g.ldo
                 : (size_t)m * g.ldo;
  };
  if constexpr (EPI == EPI_GLU) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int p = 0; p < TN / 2; ++p) {
        const int nb = n0 + wn * WN + 32 * p;      // multiple of 32
        const int na = nb + (lane & 15);
        const float ba = g.bias ? g.bias[na] : 0.f, bg = g.bias ? g.bias[na + 16] : 0.f;
        const int oc = nb / 2 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * WM + 16 * i + 4 * (lane >> 4) + r;
          if (m < g.M) {
            float a = acc[i][2 * p][r] + ba, gt = acc[i][2 * p + 1][r] + bg;
            out[orow(m) + oc] = from_f<OutT>(a * sigmoidf_(gt));
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + 16 * j + (lane & 15);
        const float bn = g.bias ? g.bias[n] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * WM + 16 * i + 4 * (lane >> 4) + r;
          if (m >= g.M) continue;
          float v = acc[i][j][r] + bn;
          if constexpr (EPI == EPI_RESID) {
            float* rp = g.resid + (size_t)m * g.ldr + n;
            *rp = *rp + g.alpha * v;
          } else {
            if constexpr (EPI == EPI_SWISH) v = swishf_(v);
            if constexpr (EPI == EPI_RELU) v = fmaxf(v, 0.f);
            if constexpr (EPI == EPI_GELU) v = geluf_(v);
            out[orow(m) + n] = from_f<OutT>(v);
            if constexpr (EPI == EPI_STORE)
              if (g.resid) g.resid[(size_t)m * g.ldr + n] = v;
          }
        }
      }
  }
}

template <typename T, typename OutT, int EPI>
static void launch_tile(const GemmArgs& g, hipStream_t s) {
  if (g.M > 1536 && g.N % 128 == 0) {
    dim3 grid(g.N / 128, (g.M + 127) / 128);
    hipLaunchKernelGGL((gemm_kernel<T, OutT, 128, 128, EPI>), grid, dim3(256), 0, s, g);
  } else {
    dim3 grid(g.N / 64, (g.M + 63) / 64);
    hipLaunchKernelGGL((gemm_kernel<T, OutT, 64, 64, EPI>), grid, dim3(256), 0, s, g);
  }
}

template <typename T, typename OutT>
static void launch_epi(const GemmArgs& g, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: launch_tile<T, OutT, EPI_STORE>(g, s); break;
    case EPI_SWISH: launch_tile<T, OutT, EPI_SWISH>(g, s); break;
    case EPI_RELU: launch_tile<T, OutT, EPI_RELU>(g, s); break;
    case EPI_GELU: launch_tile<T, OutT, EPI_GELU>(g, s); break;
    default: break;
  }
}

// Shapes are validated by the caller: N % 64 == 0, K % 64 == 0, rows of A
// and W 16-byte aligned.
void gemm(const GemmArgs& g, int epi, bool bf16_in, bool bf16_out, hipStream_t s) {
  if (g.M <= 0) return;
  const double ie = bf16_in ? 2 : 4, oe = (epi == EPI_RESID) ? 8 : (bf16_out ? 2 : 4);
  const double on = epi == EPI_GLU ? 0.5 : 1.0;
  ProfScope ps(PROF_GEMM, s, 2.0 * g.M * g.N * g.K,
               ie * ((double)g.M * g.K + (double)g.N * g.K) + oe * on * g.M * g.N);
  if (epi == EPI_RESID) {
    if (bf16_in) launch_tile<bf16_t, float, EPI_RESID>(g, s);
    else launch_tile<float, float, EPI_RESID>(g, s);
    return;
  }
  if (epi == EPI_GLU) {
    if (bf16_in) launch_tile<bf16_t, float, EPI_GLU>(g, s);
    else launch_tile<float, float, EPI_GLU>(g, s);
    return;
  }
  if (bf16_in) {
    if (bf16_out) launch_epi<bf16_t, bf16_t>(g, epi, s);
    else launch_epi<bf16_t, float>(g, epi, s);
  } else {
    if (bf16_out) launch_epi<float, bf16_t>(g, epi, s);
    else launch_epi<float, float>(g, epi, s);
  }
}

}  // namespace sf
