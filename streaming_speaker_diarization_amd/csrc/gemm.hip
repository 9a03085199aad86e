// Dense GEMM for every Linear layer of the forward: C[M,N] = A[M,K] * W[N,K]^T
// (PyTorch Linear layout, both operands K-contiguous) on MFMA, with the
// elementwise work that follows each Linear fused into the epilogue (bias,
// Swish, ReLU, GELU, GLU) or, for residual branches, written as fp32
// split-K partial sums that the following LayerNorm adds into the residual
// stream (every residual Linear of the three encoders is followed by one).
//
// Two kernels, both 256 threads = 4 waves in a 2x2 grid of 16x16 MFMA tiles:
//  * slice kernel (windows of up to a few thousand rows, the streaming case):
//    a 64x64 output tile and one K-slice of at most 512 (bf16) / 256 (fp32)
//    columns; the whole A and W slices are loaded into LDS with every global
//    load in flight at once, so a launch pays the memory latency once instead
//    of once per K tile. Longer K is split over blockIdx.z into fp32 partial
//    sums, reduced in a fixed order (deterministic) by the consumer.
//  * loop kernel (large batched windows): BMxBN tiles, BK-column K tiles
//    double-buffered through registers and LDS.
#include <utility>

#include "kernels.h"

namespace sf {

template <int EPI, typename OutT>
__device__ __forceinline__ void epi_store(const GemmArgs& g, int m, int n, float v) {
  OutT* out = static_cast<OutT*>(g.out);
  const size_t row = g.rpb ? (size_t)(m / g.rpb) * g.bstride + (size_t)(m % g.rpb) * g.ldo
                           : (size_t)m * g.ldo;
  if constexpr (EPI == EPI_SWISH) v = swishf_(v);
  if constexpr (EPI == EPI_RELU) v = fmaxf(v, 0.f);
  if constexpr (EPI == EPI_GELU) v = geluf_(v);
  out[row + n] = from_f<OutT>(v);
  if constexpr (EPI == EPI_STORE)
    if (g.resid) g.resid[(size_t)m * g.ldr + n] = v;
}

// Q/K columns go to out, V columns to the per-head transposed buffer.
template <typename OutT>
__device__ __forceinline__ void qkv_store(const GemmArgs& g, int m, int n, float v) {
  if (n < g.vcol) {
    static_cast<OutT*>(g.out)[(size_t)m * g.ldo + n] = from_f<OutT>(v);
  } else {
    const int nn = n - g.vcol, hh = nn / g.vhd, d = nn % g.vhd;
    const int bb = m / g.vrows, w = m % g.vrows, H = (g.N - g.vcol) / g.vhd;
    static_cast<OutT*>(g.vt)[((size_t)(bb * H + hh) * g.vhd + d) * g.vpitch + w] = from_f<OutT>(v);
  }
}

template <int EPI>
__device__ __forceinline__ float activate(float v) {
  if constexpr (EPI == EPI_SWISH) v = swishf_(v);
  if constexpr (EPI == EPI_RELU) v = fmaxf(v, 0.f);
  if constexpr (EPI == EPI_GELU) v = geluf_(v);
  return v;
}

// Output columns of a BN-wide tile (GLU halves them).
template <int EPI, int BN> struct TileCols { static constexpr int C = EPI == EPI_GLU ? BN / 2 : BN; };

// LDS bytes the staged epilogue needs for a BM x BN tile (fp32, padded rows).
template <int EPI, int BM, int BN>
constexpr int stage_bytes() { return BM * (TileCols<EPI, BN>::C + 4) * 4; }

// Epilogue, step 1: every wave writes its TMxTN grid of 16x16 accumulators
// (lane l: rows 4*(l/16)+r, column l%16 of each tile) with bias and
// activation applied into an fp32 tile in LDS. GLU: the weight rows were
// interleaved in blocks of 16 (value, gate), so accumulator tiles 2p and 2p+1
// hold the value and gate halves of the same 16 output columns.
template <int EPI, int BN, int TM, int TN>
__device__ __forceinline__ void stage_tile(const GemmArgs& g, const f32x4 (&acc)[TM][TN],
                                           float* cs, int n0, int wr, int wc, int lane) {
  constexpr int LDC = TileCols<EPI, BN>::C + 4;
  const int c16 = lane & 15, g4 = 4 * (lane >> 4);
  if constexpr (EPI == EPI_GLU) {
#pragma unroll
    for (int p = 0; p < TN / 2; ++p) {
      const int na = n0 + wc + 32 * p + c16;
      const float ba = g.bias ? g.bias[na] : 0.f, bg = g.bias ? g.bias[na + 16] : 0.f;
      const int oc = (wc + 32 * p) / 2 + c16;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          cs[(wr + 16 * i + g4 + r) * LDC + oc] =
              (acc[i][2 * p][r] + ba) * sigmoidf_(acc[i][2 * p + 1][r] + bg);
    }
  } else {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int c = wc + 16 * j + c16;
      const float bn = (EPI != EPI_PARTIAL && g.bias) ? g.bias[n0 + c] : 0.f;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          cs[(wr + 16 * i + g4 + r) * LDC + c] = activate<EPI>(acc[i][j][r] + bn);
    }
  }
}

template <typename OutT> struct OutVec;
template <> struct OutVec<float> {
  static constexpr int E = 4;  // elements per 16-byte store
  __device__ static void put(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct OutVec<bf16_t> {
  static constexpr int E = 8;
  __device__ static void put(bf16_t* p, const float* v) {
    uint4 u;
    u.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    u.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    u.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
    u.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
    *reinterpret_cast<uint4*>(p) = u;
  }
};

__device__ __forceinline__ bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15) == 0;
}

// Epilogue, step 2 (after a barrier): the workgroup stores the staged tile
// with 16-byte row-contiguous writes (V columns of EPI_QKV: contiguous along
// the keys of V^T). Rows past M are skipped; a chunk that is misaligned or
// crosses a stream boundary of V^T falls back to element stores.
template <int EPI, typename OutT, int BM, int BN>
__device__ __forceinline__ void store_tile(const GemmArgs& g, const float* cs, int m0, int n0,
                                           int split, int tid) {
  constexpr int C = TileCols<EPI, BN>::C;
  constexpr int LDC = C + 4;
  if constexpr (EPI == EPI_PARTIAL) {
    float* part = static_cast<float*>(g.out);
    for (int q = tid; q < BM * C / 4; q += 256) {
      const int r = q / (C / 4), c = (q % (C / 4)) * 4, m = m0 + r;
      if (m < g.M)
        *reinterpret_cast<float4*>(part + ((size_t)split * g.M + m) * g.N + n0 + c) =
            *reinterpret_cast<const float4*>(cs + r * LDC + c);
    }
    return;
  }
  constexpr int E = OutVec<OutT>::E;
  if constexpr (EPI == EPI_QKV) {
    if (n0 >= g.vcol) {  // V block: column c of the tile is one (head, dim) row of V^T
      OutT* vt = static_cast<OutT*>(g.vt);
      const int H = (g.N - g.vcol) / g.vhd;
      if (g.vrows >= BM) {
        // The tile's rows fall in at most two windows, A = m0 / vrows and A+1.
        // Keys are written in groups of 8 aligned to the window's own key
        // index w (a window of vrows % 8 != 0 rows starts off the tile's
        // 8-row grid): whole groups as vectors, the group cut by the tile's
        // edge or the window's end element by element. Within a wave, 16
        // columns x 4 consecutive groups.
        const int W = g.vrows, m1 = min(m0 + BM, g.M);
        const int bA = m0 / W, loA = m0 - bA * W, hiA = min(m1 - bA * W, W);
        const int gA0 = loA >> 3, nA = ((hiA - 1) >> 3) - gA0 + 1;
        const int hiB = m1 - (bA + 1) * W;  // rows of window A+1 in the tile
        const int nG = nA + (hiB > 0 ? ((hiB - 1) >> 3) + 1 : 0);
        constexpr int NG = (BM / 8 + 2 + 3) / 4 * 4;  // bound on groups per tile
        static_assert(C % 16 == 0, "V tile columns");
        for (int q = tid; q < C * NG; q += 256) {
          const int c = (q / 64) % (C / 16) * 16 + (q & 15);
          const int gi = (q / 64) / (C / 16) * 4 + ((q >> 4) & 3);
          if (gi >= nG) continue;
          const bool inA = gi < nA;
          const int bb = inA ? bA : bA + 1, grp = inA ? gA0 + gi : gi - nA;
          const int lo = inA ? loA : 0, hi = inA ? hiA : hiB;
          const int w0 = grp * 8, ws = max(w0, lo), we = min(w0 + 8, hi);
          const int rb = bb * W - m0;  // tile row of key 0 of window bb
          const int nn = n0 + c - g.vcol, hh = nn / g.vhd, d = nn % g.vhd;
          OutT* dst = vt + ((size_t)(bb * H + hh) * g.vhd + d) * g.vpitch + w0;
          if (ws == w0 && we == w0 + 8 && aligned16(dst)) {
#pragma unroll
            for (int e0 = 0; e0 < 8; e0 += E) {
              float v[E];
#pragma unroll
              for (int e = 0; e < E; ++e) v[e] = cs[(rb + w0 + e0 + e) * LDC + c];
              OutVec<OutT>::put(dst + e0, v);
            }
          } else {
            for (int w = ws; w < we; ++w) dst[w - w0] = from_f<OutT>(cs[(rb + w) * LDC + c]);
          }
        }
        return;
      }
      for (int q = tid; q < BM / E * C; q += 256) {
        const int c = q / (BM / E), r = (q % (BM / E)) * E, m = m0 + r;
        if (m >= g.M) continue;
        const int nn = n0 + c - g.vcol, hh = nn / g.vhd, d = nn % g.vhd;
        const int bb = m / g.vrows, w = m % g.vrows;
        OutT* dst = vt + ((size_t)(bb * H + hh) * g.vhd + d) * g.vpitch + w;
        float v[E];
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = cs[(r + e) * LDC + c];
        if (m + E <= g.M && w + E <= g.vrows && aligned16(dst)) {
          OutVec<OutT>::put(dst, v);
        } else {
          for (int e = 0; e < E && m + e < g.M; ++e) {
            const int b2 = (m + e) / g.vrows, w2 = (m + e) % g.vrows;
            vt[((size_t)(b2 * H + hh) * g.vhd + d) * g.vpitch + w2] = from_f<OutT>(v[e]);
          }
        }
      }
      return;
    }
  }
  OutT* out = static_cast<OutT*>(g.out);
  for (int q = tid; q < BM * C / E; q += 256) {
    const int r = q / (C / E), c = (q % (C / E)) * E, m = m0 + r;
    if (m >= g.M) continue;
    const size_t row = g.rpb ? (size_t)(m / g.rpb) * g.bstride + (size_t)(m % g.rpb) * g.ldo
                             : (size_t)m * g.ldo;
    const int oc = (EPI == EPI_GLU ? n0 / 2 : n0) + c;
    float v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = cs[r * LDC + c + e];
    OutT* dst = out + row + oc;
    if (aligned16(dst)) {
      OutVec<OutT>::put(dst, v);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) dst[e] = from_f<OutT>(v[e]);
    }
    if constexpr (EPI == EPI_STORE) {
      if (g.resid) {
        float* rd = g.resid + (size_t)m * g.ldr + oc;
#pragma unroll
        for (int e = 0; e < E; ++e) rd[e] = v[e];
      }
    }
  }
}

// ------------------------------------------------------------ slice kernel
template <typename T> struct SliceCfg;
template <> struct SliceCfg<bf16_t> { static constexpr int KMAX = 512; };
template <> struct SliceCfg<float> { static constexpr int KMAX = 256; };

// KS (the slice width) is a template parameter so that every thread issues a
// fixed number of unconditional 16-byte loads: rows past M read a clamped
// (valid) row and are zeroed by a select afterwards, so no load sits behind a
// branch and all of them are in flight together.
template <typename T, typename OutT, int EPI, int KS, int BM>
__global__ __launch_bounds__(256) void gemm_slice_kernel(GemmArgs g) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int LD = KS + VEC;
  constexpr int CPR = KS / VEC;
  constexpr int NCA = BM * CPR / 256;        // 16-byte chunks per thread: A
  constexpr int NCB = 64 * CPR / 256;        // and W
  constexpr int TM = BM / 32;                // 16-row MFMA tiles per wave (waves 2 x 2)
  static_assert(BM * CPR % 256 == 0 && 64 * CPR % 256 == 0, "slice width");
  using M_ = MF<T>;
  constexpr int AB = (BM + 64) * LD * (int)sizeof(T), ST = stage_bytes<EPI, BM, 64>();
  __shared__ __align__(16) char smem[AB > ST ? AB : ST];
  T* As = reinterpret_cast<T*>(smem);
  T* Bs = As + BM * LD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * 64, m0 = blockIdx.y * BM, split = blockIdx.z;
  const int k0 = split * KS;
  const T* A = static_cast<const T*>(g.A);
  const T* Wt = static_cast<const T*>(g.W);

  vec16 ra[NCA], rb[NCB];
#pragma unroll
  for (int i = 0; i < NCA; ++i) {
    const int c = tid + 256 * i, r = c / CPR, kc = (c % CPR) * VEC;
    ra[i] = *reinterpret_cast<const vec16*>(A + (size_t)min(m0 + r, g.M - 1) * g.lda + k0 + kc);
  }
#pragma unroll
  for (int i = 0; i < NCB; ++i) {
    const int c = tid + 256 * i, r = c / CPR, kc = (c % CPR) * VEC;
    rb[i] = *reinterpret_cast<const vec16*>(Wt + (size_t)(n0 + r) * g.ldw + k0 + kc);
  }
#pragma unroll
  for (int i = 0; i < NCA; ++i) {
    const int c = tid + 256 * i, r = c / CPR, kc = (c % CPR) * VEC;
    const bool live = m0 + r < g.M;
#pragma unroll
    for (int q = 0; q < 4; ++q) ra[i].w[q] = live ? ra[i].w[q] : 0u;
    *reinterpret_cast<vec16*>(&As[r * LD + kc]) = ra[i];
  }
#pragma unroll
  for (int i = 0; i < NCB; ++i) {
    const int c = tid + 256 * i, r = c / CPR, kc = (c % CPR) * VEC;
    *reinterpret_cast<vec16*>(&Bs[r * LD + kc]) = rb[i];
  }
  __syncthreads();

  f32x4 acc[TM][2];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const T* ap = &As[(wm * (BM / 2) + (lane & 15)) * LD];
  const T* bp = &Bs[(wn * 32 + (lane & 15)) * LD];
#pragma unroll 4
  for (int k = 0; k < KS; k += M_::KI) {
    typename M_::frag af[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = M_::ld(ap + 16 * i * LD + k, lane);
    typename M_::frag b0 = M_::ld(bp + k, lane), b1 = M_::ld(bp + 16 * LD + k, lane);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      acc[i][0] = M_::mma(af[i], b0, acc[i][0]);
      acc[i][1] = M_::mma(af[i], b1, acc[i][1]);
    }
  }
  __syncthreads();  // every wave is done with As/Bs: the tile is staged over them
  float* cs = reinterpret_cast<float*>(smem);
  stage_tile<EPI, 64, TM, 2>(g, acc, cs, n0, wm * (BM / 2), wn * 32, lane);
  __syncthreads();
  store_tile<EPI, OutT, BM, 64>(g, cs, m0, n0, split, tid);
}

// ------------------------------------------------------------- loop kernel
template <typename T, typename OutT, int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_loop_kernel(GemmArgs g, int ks) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int BK = sizeof(T) == 2 ? 64 : 32;
  constexpr int LDK = BK + VEC;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int CPR = BK / VEC;
  constexpr int A_IT = BM * CPR / 256;
  constexpr int B_IT = BN * CPR / 256;
  using M_ = MF<T>;
  constexpr int AB = 2 * (BM + BN) * LDK * (int)sizeof(T), ST = stage_bytes<EPI, BM, BN>();
  __shared__ __align__(16) char smem[AB > ST ? AB : ST];
  T (*As)[BM * LDK] = reinterpret_cast<T (*)[BM * LDK]>(smem);
  T (*Bs)[BN * LDK] = reinterpret_cast<T (*)[BN * LDK]>(smem + 2 * BM * LDK * sizeof(T));

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM, split = blockIdx.z;
  const T* A = static_cast<const T*>(g.A) + (size_t)split * ks;
  const T* Wt = static_cast<const T*>(g.W) + (size_t)split * ks;

  // register staging of one BK-wide K tile (plain loops, no lambdas, so the
  // arrays stay in registers)
  vec16 ra[A_IT], rb[B_IT];
#define SF_LOOP_FETCH(kt)                                                              \
  {                                                                                    \
    const int k0_ = (kt) * BK;                                                         \
    _Pragma("unroll") for (int i = 0; i < A_IT; ++i) {                                 \
      const int c = tid + i * 256, r = c / CPR, kc = (c % CPR) * VEC;                  \
      ra[i] = *reinterpret_cast<const vec16*>(A + (size_t)min(m0 + r, g.M - 1) * g.lda + \
                                              k0_ + kc);                               \
    }                                                                                  \
    _Pragma("unroll") for (int i = 0; i < B_IT; ++i) {                                 \
      const int c = tid + i * 256, r = c / CPR, kc = (c % CPR) * VEC;                  \
      rb[i] = *reinterpret_cast<const vec16*>(Wt + (size_t)(n0 + r) * g.ldw + k0_ + kc); \
    }                                                                                  \
  }
#define SF_LOOP_STASH(buf)                                                             \
  {                                                                                    \
    _Pragma("unroll") for (int i = 0; i < A_IT; ++i) {                                 \
      const int c = tid + i * 256, r = c / CPR, kc = (c % CPR) * VEC;                  \
      const bool live = m0 + r < g.M;                                                  \
      _Pragma("unroll") for (int q = 0; q < 4; ++q) ra[i].w[q] = live ? ra[i].w[q] : 0u; \
      *reinterpret_cast<vec16*>(&As[buf][r * LDK + kc]) = ra[i];                       \
    }                                                                                  \
    _Pragma("unroll") for (int i = 0; i < B_IT; ++i) {                                 \
      const int c = tid + i * 256, r = c / CPR, kc = (c % CPR) * VEC;                  \
      *reinterpret_cast<vec16*>(&Bs[buf][r * LDK + kc]) = rb[i];                       \
    }                                                                                  \
  }

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = ks / BK;
  SF_LOOP_FETCH(0)
  SF_LOOP_STASH(0)
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // the next tile (the last one again on the final iteration: unconditional
    // loads and stores keep the staging arrays in registers)
    SF_LOOP_FETCH(min(kt + 1, nk - 1))
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
    SF_LOOP_STASH(cur ^ 1)
    __syncthreads();
  }
#undef SF_LOOP_FETCH
#undef SF_LOOP_STASH
  __syncthreads();
  float* cs = reinterpret_cast<float*>(smem);
  stage_tile<EPI, BN, TM, TN>(g, acc, cs, n0, wm * WM, wn * WN, lane);
  __syncthreads();
  store_tile<EPI, OutT, BM, BN>(g, cs, m0, n0, split, tid);
}

// ----------------------------------------------------- large-M bf16 kernel
// Batched windows (tens of thousands of rows). 128 x BN tile, 4 waves in a
// 2 x 2 grid (64 x BN/2 each), K in BK-wide tiles through an NST-deep LDS
// ring filled by LDS-DMA loads (global_load_lds_dwordx4: lane l's 16 bytes
// land at the wave's LDS block base + 16 l), so the loads for tile kt+NST-1
// are in flight while tile kt is multiplied, with no register staging. A tile row is BK/8 chunks of 16
// bytes; chunk c of row r sits at chunk position c ^ (r mod BK/8) so the 16
// rows one MFMA fragment read touches spread over the banks. Rows past M load
// a clamped row: their outputs are never stored. Workgroups are mapped to
// tiles so that each XCD (dispatch round robin over 8) owns a contiguous range
// of row blocks and its L2 fetches each A row block once.
__device__ __forceinline__ void lds_dma16(const void* g, void* lds_block) {
  __builtin_amdgcn_global_load_lds(g, lds_block, 16, 0, 0);
}

// f(integral_constant<int, I>) for every I of the sequence, in order
template <typename F, int... I>
__device__ __forceinline__ void for_each_index(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

// vmcnt-only wait (expcnt / lgkmcnt left unconstrained), n < 64
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <typename OutT, int EPI, int BN, int BK, int NST>
__global__ __launch_bounds__(256) void gemm_big_kernel(GemmArgs g) {
  using M_ = MF<bf16_t>;
  constexpr int BM = 128;
  constexpr int TM = 4, TN = BN / 32;                 // 16x16 tiles per wave
  constexpr int CPR = BK / 8;                         // 16-byte chunks per tile row
  constexpr int RPB = 64 / CPR;                       // tile rows per 1 KB DMA block
  constexpr int A_BLK = BM / RPB, B_BLK = BN / RPB;
  constexpr int STAGE = (BM + BN) * BK * 2;           // bytes per ring stage
  constexpr int LOADS = (A_BLK + B_BLK) / 4;          // LDS-DMA loads per wave per stage
  static_assert((A_BLK + B_BLK) % 4 == 0, "stage split over the waves");
  constexpr int RING = NST * STAGE, ST = stage_bytes<EPI, BM, BN>();
  __shared__ __align__(16) char smem[RING > ST ? RING : ST];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware tile order (bijection over the grid): physical workgroup i runs
  // on XCD i % 8; XCD x takes logical tiles [x*q + min(x, r), ... + q + (x < r)).
  const int gx = gridDim.x, total = gx * gridDim.y;
  const int pid = blockIdx.x + gx * blockIdx.y;
  const int q8 = total / 8, r8 = total % 8, xcd = pid % 8;
  const int t = xcd * q8 + min(xcd, r8) + pid / 8;
  const int n0 = (t % gx) * BN, m0 = (t / gx) * BM;

  const char* A = static_cast<const char*>(g.A);
  const char* Wt = static_cast<const char*>(g.W);
  // this lane's row within a DMA block and the global chunk it fetches; its
  // byte offset within the operand (32 bits: the launcher keeps both operands
  // under 4 GiB) is fixed, and each K tile moves a workgroup-uniform base, so
  // the loads take a scalar base and the wave's LDS blocks scalar addresses
  const int lr = lane / CPR, lc = (lane % CPR) ^ (lr % CPR);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t goff[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int blk = wv * LOADS + j;  // A blocks first, then B blocks
    if (blk < A_BLK) {
      const int r = min(m0 + blk * RPB + lr, g.M - 1);
      goff[j] = ((uint32_t)r * (uint32_t)g.lda + lc * 8) * 2u;
    } else {
      const int r = n0 + (blk - A_BLK) * RPB + lr;
      goff[j] = ((uint32_t)r * (uint32_t)g.ldw + lc * 8) * 2u;
    }
  }
  auto issue = [&](int kt) {
    char* st = smem + (kt % NST) * STAGE;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int blk = wv * LOADS + j;
      const char* base = (blk < A_BLK ? A : Wt) + (size_t)kt * (BK * 2);
      lds_dma16(base + goff[j], st + blk * 1024);
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = g.K / BK;
#pragma unroll
  for (int p = 0; p < NST - 1; ++p)
    if (p < nk) issue(p);
  const int fr = lane & 15, fq = lane >> 4;  // fragment row, k-chunk within a 32-wide step
  for (int kt = 0; kt < nk; ++kt) {
    // tile kt's loads are this wave's oldest outstanding ones
    if constexpr (NST >= 3) {
      if (kt + NST - 2 < nk) wait_vm<(NST - 2) * LOADS>();
      else if (kt + 1 < nk) wait_vm<LOADS>();
      else wait_vm<0>();
    } else {
      wait_vm<0>();
    }
    // every wave's part of tile kt is in LDS and tile kt-1's reads are done;
    // a bare barrier: __syncthreads() would also wait for the later tiles'
    // loads still in flight
    __builtin_amdgcn_s_barrier();
    if (kt + NST - 1 < nk) issue(kt + NST - 1);
    const char* st = smem + (kt % NST) * STAGE;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int c = ks * 4 + fq;  // 16-byte chunk of the fragment's 8 k values
      M_::frag af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * 64 + 16 * i + fr;
        af[i] = *reinterpret_cast<const bf16x8_t*>(st + r * (BK * 2) + ((c ^ (r % CPR)) << 4));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * (BN / 2) + 16 * j + fr;
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(st + BM * BK * 2 + r * (BK * 2) +
                                                    ((c ^ (r % CPR)) << 4));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = M_::mma(af[i], bfr[j], acc[i][j]);
    }
  }
  if constexpr (EPI == EPI_RESID) {
    // the residual rows this thread updates, requested before the staging so
    // that they land while it runs
    constexpr int NQ = BM * BN / 4 / 256;
    float4 xr[NQ];
    float* x = static_cast<float*>(g.out);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = tid + 256 * i, r = q / (BN / 4), c = (q % (BN / 4)) * 4;
      const int m = min(m0 + r, g.M - 1);
      xr[i] = *reinterpret_cast<const float4*>(x + (size_t)m * g.ldo + n0 + c);
    }
    __syncthreads();  // the ring is reused for the staged epilogue
    float* cs = reinterpret_cast<float*>(smem);
    stage_tile<EPI, BN, TM, TN>(g, acc, cs, n0, wm * 64, wn * (BN / 2), lane);
    __syncthreads();
    constexpr int LDC = BN + 4;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = tid + 256 * i, r = q / (BN / 4), c = (q % (BN / 4)) * 4, m = m0 + r;
      if (m < g.M) {
        const float4 t = *reinterpret_cast<const float4*>(cs + r * LDC + c);
        float4 v = xr[i];
        v.x += g.ralpha * t.x;
        v.y += g.ralpha * t.y;
        v.z += g.ralpha * t.z;
        v.w += g.ralpha * t.w;
        *reinterpret_cast<float4*>(x + (size_t)m * g.ldo + n0 + c) = v;
      }
    }
    return;
  }
  __syncthreads();  // the ring is reused for the staged epilogue
  float* cs = reinterpret_cast<float*>(smem);
  stage_tile<EPI, BN, TM, TN>(g, acc, cs, n0, wm * 64, wn * (BN / 2), lane);
  __syncthreads();
  store_tile<EPI, OutT, BM, BN>(g, cs, m0, n0, 0, tid);
}

// 64-wide K tiles, double-buffered: with the 68 KB epilogue tile two
// workgroups fit on a CU, which measured faster than deeper rings with one
#define SF_BIG_BK 64
#define SF_BIG_NST 2

// ------------------------------------------------ slice kernel, bf16 form
// Same tiling and K-slice as gemm_slice_kernel, but the slice arrives by
// LDS-DMA in 64-wide K phases (every phase's loads issued at once, no register
// staging): the MFMAs of phase p run while phases p+1.. are still landing.
// Each 64-wide phase row is 8 chunks of 16 bytes, chunk c of row r stored at
// position c ^ (r & 7); one 1 KB DMA block holds 8 rows.
// DW: the GLU + depthwise-conv epilogue (see gemm_glu_dwconv): rows
// m0-4 .. m0+BM-5 are computed, rows m0 .. m0+BM-9 written.
template <typename OutT, int EPI, int KS, int BM, bool DW = false>
__global__ __launch_bounds__(256) void gemm_slice_dma_kernel(GemmArgs g) {
  using M_ = MF<bf16_t>;
  constexpr int NPH = KS / 64;                  // K phases
  constexpr int PH = (BM + 64) * 128;           // bytes per phase (A rows, then W rows)
  constexpr int LOADS = (BM + 64) / 8 / 4;      // DMA blocks per wave per phase
  constexpr int TM = BM / 32;                   // 16-row MFMA tiles per wave (waves 2 x 2)
  static_assert(KS % 64 == 0 && (BM + 64) % 32 == 0, "slice shape");
  constexpr int AB = NPH * PH, ST = stage_bytes<EPI, BM, 64>();
  __shared__ __align__(16) char smem[AB > ST ? AB : ST];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  static_assert(!DW || EPI == EPI_GLU, "fused depthwise conv epilogue");
  constexpr int DW_OUT = BM - 8;  // rows written by the depthwise-conv epilogue
  const int n0 = blockIdx.x * 64, m0 = blockIdx.y * (DW ? DW_OUT : BM), split = blockIdx.z;
  const int mc = DW ? m0 - 4 : m0;  // first computed row
  const int k0 = split * KS;
  const bf16_t* A = static_cast<const bf16_t*>(g.A);
  const bf16_t* Wt = static_cast<const bf16_t*>(g.W);

  const int lr = lane >> 3, lc = (lane & 7) ^ lr;  // row in a DMA block, chunk fetched
#pragma unroll
  for (int p = 0; p < NPH; ++p) {
    char* ph = smem + p * PH;
    const int kk = k0 + p * 64 + lc * 8;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int blk = wave * LOADS + j;  // A blocks first, then W blocks
      if (blk < BM / 8) {
        const int r = min(max(mc + blk * 8 + lr, 0), g.M - 1);
        lds_dma16(A + (size_t)r * g.lda + kk, ph + blk * 1024);
      } else {
        const int r = n0 + (blk - BM / 8) * 8 + lr;
        lds_dma16(Wt + (size_t)r * g.ldw + kk, ph + blk * 1024);
      }
    }
  }

  f32x4 acc[TM][2];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fq = lane >> 4;
  auto phase = [&](auto pc) {
    constexpr int p = decltype(pc)::value;
    wait_vm<(NPH - 1 - p) * LOADS>();  // this wave's loads of phase p have landed
    __builtin_amdgcn_s_barrier();       // and every other wave's
    const char* ph = smem + p * PH;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = ks * 4 + fq;
      M_::frag af[TM], b0, b1;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * (BM / 2) + 16 * i + fr;
        af[i] = *reinterpret_cast<const bf16x8_t*>(ph + r * 128 + ((c ^ (r & 7)) << 4));
      }
      {
        const int r0 = BM + wn * 32 + fr, r1 = r0 + 16;
        b0 = *reinterpret_cast<const bf16x8_t*>(ph + r0 * 128 + ((c ^ (r0 & 7)) << 4));
        b1 = *reinterpret_cast<const bf16x8_t*>(ph + r1 * 128 + ((c ^ (r1 & 7)) << 4));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        acc[i][0] = M_::mma(af[i], b0, acc[i][0]);
        acc[i][1] = M_::mma(af[i], b1, acc[i][1]);
      }
    }
  };
  for_each_index(phase, std::make_integer_sequence<int, NPH>{});
  __syncthreads();  // every wave is done with the slice: the tile is staged over it
  float* cs = reinterpret_cast<float*>(smem);
  stage_tile<EPI, 64, TM, 2>(g, acc, cs, n0, wm * (BM / 2), wn * 32, lane);
  __syncthreads();
  if constexpr (!DW) {
    store_tile<EPI, OutT, BM, 64>(g, cs, m0, n0, split, tid);
  } else {
    // out[m][ch] = swish(sc * sum_t w[ch][t] glu[m+t-4][ch] + sh) for the
    // DW_OUT rows and 32 GLU channels of this tile; cs row i holds row mc + i,
    // taps whose frame leaves [0, dw_nvalid) of the row's stream are zero (the
    // same sum order as dwconv_time_kernel)
    constexpr int LDC = 32 + 4, RPT = DW_OUT / 8;
    const int c = tid & 31, r0 = (tid >> 5) * RPT, ch = n0 / 2 + c;
    float w9[9];
#pragma unroll
    for (int t = 0; t < 9; ++t) w9[t] = g.dw_w9[ch * 9 + t];
    const float sc = g.dw_sc[ch], sh = g.dw_sh[ch];
    const int nvv = g.dw_nv ? *g.dw_nv : g.dw_nvalid;
    int fr = (m0 + r0) % g.dw_W;
    bf16_t* out = static_cast<bf16_t*>(g.out);
#pragma unroll
    for (int r = r0; r < r0 + RPT; ++r) {
      const int m = m0 + r;
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < 9; ++t) {
        const int tt = fr + t - 4;
        acc += (tt >= 0 && tt < nvv) ? w9[t] * cs[(r + t) * LDC + c] : 0.f;
      }
      if (m < g.M) out[(size_t)m * g.ldo + ch] = f2bf(swishf_(sc * acc + sh));
      fr = fr + 1 == g.dw_W ? 0 : fr + 1;
    }
  }
}

// ------------------------------------------------- split-K reduce + epilogue
// v = sum_s part[s][m][n] (in split order) + bias[n], then the epilogue.
template <typename OutT, int EPI>
__global__ __launch_bounds__(256) void splitk_epi_kernel(GemmArgs g, const float* part, int ns) {
  const int m = blockIdx.x;
  const int ncol = EPI == EPI_GLU ? g.N / 2 : g.N;
  for (int c = threadIdx.x; c < ncol; c += 256) {
    auto red = [&](int n) {  // slices summed in order; the first 16 loaded at once
      float pv[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) pv[s] = s < ns ? part[((size_t)s * g.M + m) * g.N + n] : 0.f;
      float v = 0.f;
#pragma unroll
      for (int s = 0; s < 16; ++s)
        if (s < ns) v += pv[s];
      for (int s = 16; s < ns; ++s) v += part[((size_t)s * g.M + m) * g.N + n];
      return v + (g.bias ? g.bias[n] : 0.f);
    };
    if constexpr (EPI == EPI_GLU) {
      const int na = (c / 16) * 32 + (c % 16);
      OutT* out = static_cast<OutT*>(g.out);
      out[(size_t)m * g.ldo + c] = from_f<OutT>(red(na) * sigmoidf_(red(na + 16)));
    } else if constexpr (EPI == EPI_QKV) {
      qkv_store<OutT>(g, m, c, red(c));
    } else {
      epi_store<EPI, OutT>(g, m, c, red(c));
    }
  }
}

// ---------------------------------------------------------------- dispatch
// The K slicing depends only on K and the operand type (never on M), and
// both kernels accumulate a slice in the same k order, so a row's result is
// bit-identical whatever the window or batch size.
template <typename T>
static bool slice_ok(int ks) {
  return sizeof(T) == 2 ? (ks == 512 || ks == 384 || ks == 256 || ks == 192 || ks == 128 || ks == 64)
                        : (ks == 256 || ks == 192 || ks == 128 || ks == 64);
}

template <typename T>
static int n_slices(int K) {
  constexpr int KMAX = SliceCfg<T>::KMAX;
  int ns = (K + KMAX - 1) / KMAX;
  while (K % ns != 0 || !slice_ok<T>(K / ns)) ++ns;
  return ns;
}

// Residual-branch Linears (bf16, fp32 partials summed by the LayerNorm that
// follows) are split over K more finely when N is narrow, so that a window of
// a few hundred rows still fills about 32 tiles x slices per 64-row block:
// the largest slice count up to that target whose slice width is supported.
// Depends on K and N only, never on M.
template <typename T>
static int partial_slices(int K, int N) {
  const int base = n_slices<T>(K);
  if (sizeof(T) != 2) return base;
  const int target = 32 / std::max(1, N / 64);
  for (int ns = std::max(base, target); ns > base; --ns)
    if (K % ns == 0 && slice_ok<T>(K / ns)) return ns;
  return base;
}

// algorithmic work of the gemm() call being launched (for profiling)
static thread_local double g_flops = 0, g_bytes = 0;

// 64-row tiles, or 32-row tiles when 64-row ones would leave more than half
// of the 256 CUs idle (the tile height does not change any result: every
// output element accumulates the same K slice in the same order).
#ifndef SF_SLICE_DMA
#define SF_SLICE_DMA 1
#endif
template <typename T, typename OutT, int EPI, int KS>
static void slice_launch(const GemmArgs& g, int ns, hipStream_t s) {
  const int tiles64 = g.N / 64 * ((g.M + 63) / 64) * ns;
  if constexpr (sizeof(T) == 2 && KS % 64 == 0 && SF_SLICE_DMA) {
    if (tiles64 < 128)
      klaunch(PROF_GEMM, g_flops, g_bytes, gemm_slice_dma_kernel<OutT, EPI, KS, 32>,
              dim3(g.N / 64, (g.M + 31) / 32, ns), dim3(256), s, g);
    else
      klaunch(PROF_GEMM, g_flops, g_bytes, gemm_slice_dma_kernel<OutT, EPI, KS, 64>,
              dim3(g.N / 64, (g.M + 63) / 64, ns), dim3(256), s, g);
    return;
  }
  if (tiles64 < 128) {
    dim3 grid(g.N / 64, (g.M + 31) / 32, ns);
    klaunch(PROF_GEMM, g_flops, g_bytes, gemm_slice_kernel<T, OutT, EPI, KS, 32>, grid, dim3(256),
            s, g);
  } else {
    dim3 grid(g.N / 64, (g.M + 63) / 64, ns);
    klaunch(PROF_GEMM, g_flops, g_bytes, gemm_slice_kernel<T, OutT, EPI, KS, 64>, grid, dim3(256),
            s, g);
  }
}

// gemm_big_kernel addresses its operands with 32-bit byte offsets
static bool big_offsets_fit(const GemmArgs& g) {
  return (uint64_t)g.M * g.lda * 2 < (1ull << 32) && (uint64_t)g.N * g.ldw * 2 < (1ull << 32);
}

template <typename T, typename OutT, int EPI>
static void launch_kernel(const GemmArgs& g, int ns, hipStream_t s) {
  const int ks = g.K / ns;
  if (g.M <= SLICE_MAX_ROWS) {
    switch (ks) {
      case 64: slice_launch<T, OutT, EPI, 64>(g, ns, s); break;
      case 128: slice_launch<T, OutT, EPI, 128>(g, ns, s); break;
      case 192: slice_launch<T, OutT, EPI, 192>(g, ns, s); break;
      case 256: slice_launch<T, OutT, EPI, 256>(g, ns, s); break;
      default:
        if constexpr (sizeof(T) == 2) {
          if (ks == 384) slice_launch<T, OutT, EPI, 384>(g, ns, s);
          else slice_launch<T, OutT, EPI, 512>(g, ns, s);
        }
    }
  } else if (sizeof(T) == 2 && ns == 1 && g.K % SF_BIG_BK == 0 && g.N % 64 == 0 &&
             big_offsets_fit(g)) {
    if constexpr (sizeof(T) == 2) {
      if (g.N % 128 == 0)
        klaunch(PROF_GEMM, g_flops, g_bytes, gemm_big_kernel<OutT, EPI, 128, SF_BIG_BK, SF_BIG_NST>,
                dim3(g.N / 128, (g.M + 127) / 128), dim3(256), s, g);
      else
        klaunch(PROF_GEMM, g_flops, g_bytes, gemm_big_kernel<OutT, EPI, 64, SF_BIG_BK, SF_BIG_NST>,
                dim3(g.N / 64, (g.M + 127) / 128), dim3(256), s, g);
    }
  } else if (g.M > 1536 && g.N % 128 == 0) {
    dim3 grid(g.N / 128, (g.M + 127) / 128, ns);
    klaunch(PROF_GEMM, g_flops, g_bytes, gemm_loop_kernel<T, OutT, 128, 128, EPI>, grid, dim3(256), s,
            g, ks);
  } else {
    dim3 grid(g.N / 64, (g.M + 63) / 64, ns);
    klaunch(PROF_GEMM, g_flops, g_bytes, gemm_loop_kernel<T, OutT, 64, 64, EPI>, grid, dim3(256), s,
            g, ks);
  }
}

template <typename T, typename OutT, int EPI>
static int launch(const GemmArgs& g, hipStream_t s) {
  // Windows of a few thousand rows: K slices as above (at most 512 wide; finer
  // for narrow residual branches). Larger problems fill the GPU with row tiles
  // alone and run the whole K in one loop. The choice depends on the problem
  // size, not on its content: within each regime a row's result does not
  // depend on how many rows share the launch.
  const int ns = g.M > SLICE_MAX_ROWS ? 1
                 : EPI == EPI_PARTIAL ? partial_slices<T>(g.K, g.N) : n_slices<T>(g.K);
  if (ns == 1 || EPI == EPI_PARTIAL) {
    if (ns > 1 && ns > g.max_split) return -1;
    launch_kernel<T, OutT, EPI>(g, ns, s);
    return EPI == EPI_PARTIAL ? ns : 1;
  }
  if (!g.part || ns > g.max_split) return -1;
  GemmArgs p = g;
  p.out = g.part;
  launch_kernel<T, float, EPI_PARTIAL>(p, ns, s);
  g_flops = g_bytes = 0;  // the reduction launch carries no extra algorithmic work
  klaunch(PROF_GEMM, 0.0, 0.0, splitk_epi_kernel<OutT, EPI>, dim3(g.M), dim3(256), s, g,
          static_cast<const float*>(g.part), ns);
  return 1;
}

template <typename T, typename OutT>
static int launch_epi(const GemmArgs& g, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch<T, OutT, EPI_STORE>(g, s);
    case EPI_SWISH: return launch<T, OutT, EPI_SWISH>(g, s);
    case EPI_RELU: return launch<T, OutT, EPI_RELU>(g, s);
    case EPI_GELU: return launch<T, OutT, EPI_GELU>(g, s);
    case EPI_QKV: return launch<T, OutT, EPI_QKV>(g, s);
    default: return 0;
  }
}

// Shapes are validated by the caller: N % 64 == 0, K % 64 == 0, rows of A
// and W 16-byte aligned. Returns the number of partial slices written for
// EPI_PARTIAL (1 otherwise), or -1 (nothing launched) when the partial-sum
// scratch is missing or too small.
static thread_local bool g_gemm_failed = false;

bool take_gemm_failure() {
  const bool f = g_gemm_failed;
  g_gemm_failed = false;
  return f;
}

void flag_launch_failure() { g_gemm_failed = true; }

static int checked(int r) {
  if (r < 0) g_gemm_failed = true;
  return r;
}

int gemm_glu_dwconv(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return 1;
  if (g.M > SLICE_MAX_ROWS || g.K != 512 || g.N % 64 || !g.dw_w9 || g.dw_W <= 0) {
    g_gemm_failed = true;
    return -1;
  }
  g_flops = 2.0 * g.M * g.N * g.K + 2.0 * 9 * g.M * (g.N / 2);
  g_bytes = 2.0 * g.M * g.K + 2.0 * g.N * g.K + 2.0 * g.M * (g.N / 2);
  klaunch(PROF_GEMM, g_flops, g_bytes, gemm_slice_dma_kernel<bf16_t, EPI_GLU, 512, 32, true>,
          dim3(g.N / 64, (g.M + 23) / 24, 1), dim3(256), s, g);
  return 1;
}

int gemm_resid(const GemmArgs& g, hipStream_t s) {
  if (g.M <= SLICE_MAX_ROWS || g.K % SF_BIG_BK || g.N % 64 || g.K <= 0 || !big_offsets_fit(g))
    return -1;
  // 128 x 64 tiles: the N = 512 branches then make about three rounds of
  // workgroups over the CUs rather than one and a half
  klaunch(PROF_GEMM, 2.0 * g.M * g.N * g.K,
          2.0 * ((double)g.M * g.K + (double)g.N * g.K) + 8.0 * g.M * g.N,
          gemm_big_kernel<float, EPI_RESID, 64, SF_BIG_BK, SF_BIG_NST>,
          dim3(g.N / 64, (g.M + 127) / 128), dim3(256), s, g);
  return 1;
}

int gemm(const GemmArgs& g, int epi, bool bf16_in, bool bf16_out, hipStream_t s) {
  if (g.M <= 0) return 1;
  const double ie = bf16_in ? 2 : 4, oe = (epi == EPI_PARTIAL) ? 4 : (bf16_out ? 2 : 4);
  const double on = epi == EPI_GLU ? 0.5 : 1.0;
  g_flops = 2.0 * g.M * g.N * g.K;
  g_bytes = ie * ((double)g.M * g.K + (double)g.N * g.K) + oe * on * g.M * g.N;
  if (epi == EPI_PARTIAL)
    return checked(bf16_in ? launch<bf16_t, float, EPI_PARTIAL>(g, s)
                           : launch<float, float, EPI_PARTIAL>(g, s));
  if (epi == EPI_GLU)
    return checked(!bf16_in    ? launch<float, float, EPI_GLU>(g, s)
                   : bf16_out ? launch<bf16_t, bf16_t, EPI_GLU>(g, s)
                              : launch<bf16_t, float, EPI_GLU>(g, s));
  if (bf16_in)
    return checked(bf16_out ? launch_epi<bf16_t, bf16_t>(g, epi, s) : launch_epi<bf16_t, float>(g, epi, s));
  return checked(bf16_out ? launch_epi<float, bf16_t>(g, epi, s) : launch_epi<float, float>(g, epi, s));
}

}  // namespace sf
