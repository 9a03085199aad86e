// Memory-bound kernels of the forward: LayerNorm, the conformer's depthwise
// time convolution, the log-mel frontend, the strided 2-D convolutions of the
// 8x subsampling, frame stacking, the speaker heads and the small state
// copies of the streaming window. All are coalesced along the feature axis.
#include "kernels.h"

namespace sf {

// ------------------------------------------------------------- LayerNorm
// One wave per row; statistics in fp32 (two passes over registers). The
// residual partials are summed in slice order, so the result does not depend
// on scheduling.
// Columns per lane: VW consecutive columns (16-byte accesses) at
// VW*lane + 64*VW*i when D is a multiple of 256, else single columns.
template <typename T, int D, int NS>
__global__ __launch_bounds__(256) void ln_kernel(LnArgs a) {
  constexpr int PER = D / 64;
  constexpr int VW = D % 256 == 0 ? 4 : 1;
  constexpr int NV = PER / VW;
  const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= a.M) return;
  auto col = [&](int i) { return VW * lane + 64 * VW * (i / VW) + i % VW; };
  auto ld = [&](const float* p, float* dst) {  // this lane's PER columns of a row
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if constexpr (VW == 4) {
        const float4 f = *reinterpret_cast<const float4*>(p + 4 * lane + 256 * j);
        dst[4 * j] = f.x; dst[4 * j + 1] = f.y; dst[4 * j + 2] = f.z; dst[4 * j + 3] = f.w;
      } else {
        dst[j] = p[lane + 64 * j];
      }
    }
  };
  auto st = [&](float* p, const float* src) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if constexpr (VW == 4)
        *reinterpret_cast<float4*>(p + 4 * lane + 256 * j) =
            make_float4(src[4 * j], src[4 * j + 1], src[4 * j + 2], src[4 * j + 3]);
      else
        p[lane + 64 * j] = src[j];
    }
  };
  float v[PER];
  float* xr = a.x + (size_t)row * D;
  const float* xin = (a.x_in ? a.x_in : a.x) + (size_t)row * D;
  // every load of the row (residual + NS partial slices) and of the LayerNorm
  // parameters is issued before use
  float pp[NS > 0 ? NS : 1][PER];
  ld(xin, v);
  float gv1[PER], bv1[PER], gv2[PER], bv2[PER];
  ld(a.g1, gv1);
  ld(a.b1, bv1);
  if (a.g2) {
    ld(a.g2, gv2);
    ld(a.b2, bv2);
  }
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) ld(a.part + ((size_t)sp * a.M + row) * D, pp[sp]);
  if constexpr (NS > 0) {
    float pb[PER];
    ld(a.pbias, pb);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      float t = 0.f;
#pragma unroll
      for (int sp = 0; sp < NS; ++sp) t += pp[sp][i];
      v[i] += a.alpha * (t + pb[i]);
    }
  }
  if (a.x_mode == 1) st(xr, v);
  auto norm = [&](const float* gv, const float* bv) {
    float sm = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) sm += v[i];
    const float mean = wave_sum(sm) * (1.0f / D);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) { v[i] -= mean; q += v[i] * v[i]; }
    const float rstd = 1.0f / sqrtf(wave_sum(q) * (1.0f / D) + 1e-5f);
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = v[i] * rstd * gv[i] + bv[i];
  };
  norm(gv1, bv1);
  if (a.x_mode == 2) st(xr, v);
  if (a.g2) norm(gv2, bv2);
  if (a.y_act) {
    T* y = static_cast<T*>(a.y_act) + (size_t)row * D;
    if constexpr (VW == 4 && sizeof(T) == 2) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        u16x4 u;
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = f2bf(v[4 * j + e]);
        *reinterpret_cast<u16x4*>(y + 4 * lane + 256 * j) = u;
      }
    } else if constexpr (VW == 4) {
      st(reinterpret_cast<float*>(y), v);
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) y[col(i)] = from_f<T>(v[i]);
    }
  }
}

template <typename T, int D>
static void ln_launch(const LnArgs& a, dim3 grid, dim3 block, hipStream_t s, double by) {
  switch (a.part ? a.nsplit : 0) {
    case 0: klaunch(PROF_LN, 0.0, by, ln_kernel<T, D, 0>, grid, block, s, a); break;
    case 1: klaunch(PROF_LN, 0.0, by, ln_kernel<T, D, 1>, grid, block, s, a); break;
    case 2: klaunch(PROF_LN, 0.0, by, ln_kernel<T, D, 2>, grid, block, s, a); break;
    case 3: klaunch(PROF_LN, 0.0, by, ln_kernel<T, D, 3>, grid, block, s, a); break;
    case 4: klaunch(PROF_LN, 0.0, by, ln_kernel<T, D, 4>, grid, block, s, a); break;
    case 6: klaunch(PROF_LN, 0.0, by, ln_kernel<T, D, 6>, grid, block, s, a); break;
    case 8: klaunch(PROF_LN, 0.0, by, ln_kernel<T, D, 8>, grid, block, s, a); break;
    default: break;  // rejected by layernorm()
  }
}

#ifndef SF_LN_ROWS1
#define SF_LN_ROWS1 1024
#endif
void layernorm(const LnArgs& a, bool bf16, hipStream_t s) {
  if (a.M <= 0) return;
  const int ns = a.part ? a.nsplit : 0;
  if (ns < 0 || ns == 5 || ns == 7 || ns > 8 || (ns > 0 && !a.pbias)) {
    flag_launch_failure();
    return;
  }
  const double by = (double)a.M * a.D * (4.0 + 4.0 * ns + (a.x_mode ? 4.0 : 0.0) +
                                           (a.y_act ? (bf16 ? 2.0 : 4.0) : 0.0));
  // one row per wave; single-wave workgroups while that still leaves the
  // grid within a few rounds of the 256 CUs (the loads of a row are then
  // spread over more CUs), four-wave workgroups beyond
  const int rpb = a.M <= SF_LN_ROWS1 ? 1 : 4;
  const dim3 grid((a.M + rpb - 1) / rpb), block(64 * rpb);
  if (bf16) {
    if (a.D == 512) ln_launch<bf16_t, 512>(a, grid, block, s, by);
    else ln_launch<bf16_t, 192>(a, grid, block, s, by);
  } else {
    if (a.D == 512) ln_launch<float, 512>(a, grid, block, s, by);
    else ln_launch<float, 192>(a, grid, block, s, by);
  }
}

// ------------------------------------------- conformer depthwise conv (k=9)
// out[t,c] = swish(scale[c] * sum_k w[c,k] g[t+k-4,c] + shift[c]); rows at or
// beyond n_valid (and outside the window) count as zero. BatchNorm and the
// conv bias are folded into scale/shift. One workgroup = R frames of one
// stream; a thread owns 4 channels and keeps the R + 8 input rows of them in
// registers (each input row loaded once). R = 4 for one or a few windows
// (enough workgroups to fill the chip), 16 for batched windows (1.5 rows read
// per row written instead of 3). The GLU output arrives as TI (fp32, or bf16
// in batched bf16 windows).
template <typename TI, typename T, int R>
__global__ __launch_bounds__(128) void dwconv_time_kernel(const TI* glu, int W, int n_valid_h,
                                                          const int* nv, const float* w9,
                                                          const float* sc, const float* sh, T* out) {
  const int n_valid = nv ? *nv : n_valid_h;
  // XCD-aware order (bijection over the grid): physical workgroup i runs on
  // XCD i % 8, and XCD x takes a contiguous range of (stream, row block), so
  // the halo rows that neighbouring blocks share come from one L2
  int t0, b;
  {
    const int gx = gridDim.x, total = gx * gridDim.y;
    const int pid = blockIdx.x + gx * blockIdx.y;
    const int q8 = total / 8, r8 = total % 8, xcd = pid % 8;
    const int t = xcd * q8 + min(xcd, r8) + pid / 8;
    t0 = (t % gx) * R;
    b = t / gx;
  }
  const int c = threadIdx.x * 4;
  const TI* gb = glu + (size_t)b * W * 512 + c;
  float4 x[R + 8];
#pragma unroll
  for (int j = 0; j < R + 8; ++j) {
    const TI* src = gb + (size_t)min(max(t0 + j - 4, 0), W - 1) * 512;
    if constexpr (sizeof(TI) == 4) {
      x[j] = *reinterpret_cast<const float4*>(src);
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(src);
      x[j] = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                         __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    }
  }
  float4 wk[9];  // w[c..c+3][k] for tap k, from the [c][9] layout
  {
    float wr[36];
#pragma unroll
    for (int q = 0; q < 9; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(w9 + c * 9 + 4 * q);
      wr[4 * q] = v.x; wr[4 * q + 1] = v.y; wr[4 * q + 2] = v.z; wr[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int k = 0; k < 9; ++k) wk[k] = make_float4(wr[k], wr[9 + k], wr[18 + k], wr[27 + k]);
  }
  const float4 s4 = *reinterpret_cast<const float4*>(sc + c);
  const float4 h4 = *reinterpret_cast<const float4*>(sh + c);
  // every tap of every row of the block inside [0, n_valid): no masking
  const bool interior = t0 >= 4 && t0 + R + 4 <= n_valid;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + r;
    if (t >= W) break;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (interior) {
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        const float4 v = x[r + k];
        acc.x = fmaf(wk[k].x, v.x, acc.x);
        acc.y = fmaf(wk[k].y, v.y, acc.y);
        acc.z = fmaf(wk[k].z, v.z, acc.z);
        acc.w = fmaf(wk[k].w, v.w, acc.w);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        const int tt = t + k - 4;
        const bool live = tt >= 0 && tt < n_valid;
        const float4 v = x[r + k];
        acc.x += live ? wk[k].x * v.x : 0.f;
        acc.y += live ? wk[k].y * v.y : 0.f;
        acc.z += live ? wk[k].z * v.z : 0.f;
        acc.w += live ? wk[k].w * v.w : 0.f;
      }
    }
    float y[4] = {swishf_(s4.x * acc.x + h4.x), swishf_(s4.y * acc.y + h4.y),
                  swishf_(s4.z * acc.z + h4.z), swishf_(s4.w * acc.w + h4.w)};
    T* o = out + ((size_t)b * W + t) * 512 + c;
    if constexpr (sizeof(T) == 2) {
      uint2 u;
      u.x = (uint32_t)f2bf(y[0]) | ((uint32_t)f2bf(y[1]) << 16);
      u.y = (uint32_t)f2bf(y[2]) | ((uint32_t)f2bf(y[3]) << 16);
      *reinterpret_cast<uint2*>(o) = u;
    } else {
      *reinterpret_cast<float4*>(o) = make_float4(y[0], y[1], y[2], y[3]);
    }
  }
}

void dwconv_time(const void* glu, bool glu_bf16, int B, int W, int n_valid, const int* nv,
                 const float* w9, const float* sc, const float* sh, void* out, bool bf16,
                 hipStream_t s) {
  if (W <= 0) return;
  const double fl = 2.0 * 9 * 512 * B * W,
               by = (double)B * W * 512 * ((glu_bf16 ? 2.0 : 4.0) + (bf16 ? 2 : 4));
  auto go = [&](auto rows) {
    constexpr int R = decltype(rows)::value;
    dim3 grid((W + R - 1) / R, B);
    if (glu_bf16 && bf16)
      klaunch(PROF_CONV, fl, by, dwconv_time_kernel<bf16_t, bf16_t, R>, grid, dim3(128), s,
              static_cast<const bf16_t*>(glu), W, n_valid, nv, w9, sc, sh,
              static_cast<bf16_t*>(out));
    else if (bf16)
      klaunch(PROF_CONV, fl, by, dwconv_time_kernel<float, bf16_t, R>, grid, dim3(128), s,
              static_cast<const float*>(glu), W, n_valid, nv, w9, sc, sh,
              static_cast<bf16_t*>(out));
    else
      klaunch(PROF_CONV, fl, by, dwconv_time_kernel<float, float, R>, grid, dim3(128), s,
              static_cast<const float*>(glu), W, n_valid, nv, w9, sc, sh,
              static_cast<float*>(out));
  };
  if ((size_t)B * W > 4096) go(std::integral_constant<int, 16>{});
  else go(std::integral_constant<int, 4>{});
}

// ------------------------------------------------------------ log-mel
// Table block (floats): [0,512) cos(2 pi m/512), [512,1024) sin(2 pi m/512),
// [1024,1424) analysis window (periodic Hann 400), then per mel band m:
// lo[m], cnt[m] (as floats) at 1424+2m, and weights at 1680 + m*MELW.
#define MEL_TAB_LO 1424
#define MEL_TAB_W 1680
#define MELW 32
// Frame t covers samples 160t-200 ... 160t+199, the non-zero part of the
// centred 512-point frame (window sample n at frame position n + 56); samples
// outside [0, n_total) are zero. One workgroup per frame: the windowed frame
// goes to LDS in bit-reversed order, a radix-2 decimation-in-time FFT (9
// stages, one butterfly per thread each) gives the 257 bins, then |X|^2, the
// sparse mel sums and log(x + 2^-24).
__global__ __launch_bounds__(256) void logmel_kernel(const float* audio, long long a_bstride,
                                                     long long ring_mask, long long n_total,
                                                     long long t0, int nfr, const float* tab,
                                                     float* mel, long long m_bstride) {
  __shared__ float xr[512], xi[512];
  __shared__ float tc[256], ts[256];
  __shared__ float pw[257];
  const int tid = threadIdx.x, b = blockIdx.y, fr = blockIdx.x;
  const float* ab = audio + (size_t)b * a_bstride;
  tc[tid] = tab[tid];
  ts[tid] = tab[512 + tid];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = tid + 256 * h, n = p - 56;  // frame position, window sample
    const long long smp = 160 * (t0 + fr) - 256 + p;
    const long long sc = smp < 0 ? 0 : (smp >= n_total ? n_total - 1 : smp);
    const float v = ab[sc & ring_mask];
    const bool live = n >= 0 && n < 400 && smp >= 0 && smp < n_total;
    const int q = (int)(__brev((unsigned)p) >> 23);
    xr[q] = live ? v * tab[1024 + n] : 0.f;
    xi[q] = 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int st = 0; st < 9; ++st) {
    const int half = 1 << st, pos = tid & (half - 1);
    const int i0 = ((tid >> st) << (st + 1)) + pos, i1 = i0 + half;
    const int k = pos << (8 - st);  // twiddle exp(-2 pi i pos / (2 half)) = exp(-2 pi i k / 512)
    const float c = tc[k], sn = ts[k];
    const float ar = xr[i0], ai = xi[i0], br = xr[i1], bi = xi[i1];
    const float tr = br * c + bi * sn, ti = bi * c - br * sn;
    __syncthreads();
    xr[i0] = ar + tr;
    xi[i0] = ai + ti;
    xr[i1] = ar - tr;
    xi[i1] = ai - ti;
    __syncthreads();
  }
  pw[tid] = xr[tid] * xr[tid] + xi[tid] * xi[tid];
  if (tid == 0) pw[256] = xr[256] * xr[256] + xi[256] * xi[256];
  __syncthreads();
  if (tid < 128 && fr < nfr) {
    const int m = tid;
    const int lo = (int)tab[MEL_TAB_LO + 2 * m], cnt = (int)tab[MEL_TAB_LO + 2 * m + 1];
    float acc = 0.f;
    for (int i = 0; i < cnt; ++i) acc += tab[MEL_TAB_W + m * MELW + i] * pw[lo + i];
    mel[(size_t)b * m_bstride + (size_t)fr * 128 + m] = logf(acc + 5.9604644775390625e-8f);
  }
}

void logmel(const float* audio, long long a_bstride, long long ring_mask, long long n_total,
            long long t0, int nfr, int B, const float* tab, float* mel, long long m_bstride,
            hipStream_t s) {
  if (nfr <= 0) return;
  dim3 grid(nfr, B);
  klaunch(PROF_FRONTEND, (double)B * nfr * (2.0 * 2 * 400 * 257 + 2.0 * 257 * 2),
          (double)B * nfr * (160 * 4 + 128 * 4), logmel_kernel, grid, dim3(256), s, audio,
          a_bstride, ring_mask, n_total, (long long)t0, nfr, tab, mel, m_bstride);
}

// ------------------------------------------------ 8x ConvSubsampling parts
// Layouts are channels-last: (rows, freq, 256). Row indices are absolute
// within the utterance; a buffer holds rows [base, base+n). Input rows
// outside [0, len_in) are the convolution's zero padding.
// conv0: one workgroup = FB output frequencies of one output row of one
// stream, thread = output channel; the 3 x (2 FB + 1) input patch they share
// is staged in LDS once. Large batches take FB = 16 (fewer, longer
// workgroups); a single stream keeps one frequency per workgroup so that its
// few rows still spread over the chip. Every output is computed the same way
// either way.
template <int FB>
__global__ __launch_bounds__(256) void conv0_kernel(const float* mel, long long mel_bstride,
                                                    int mel_base, int T, float* out,
                                                    long long out_bstride, int o_base,
                                                    const float* w, const float* bias) {
  constexpr int NJ = 2 * FB + 1;
  __shared__ float xs[3][NJ];
  const int o = blockIdx.x / (64 / FB), f0 = (blockIdx.x % (64 / FB)) * FB;
  const int b = blockIdx.y, c = threadIdx.x;
  const float* mb = mel + (size_t)b * mel_bstride;
  const int r0 = 2 * (o_base + o) - 1;
  const int rlo = max(r0, max(0, mel_base)), rhi = min(r0 + 2, T - 1);
  auto in_at = [&](int a, int j) {
    const int r = min(max(r0 + a, rlo), rhi), col = min(max(2 * f0 - 1 + j, 0), 127);
    return mb[(size_t)(r - mel_base) * 128 + col];
  };
  float x1[3][3];  // FB = 1: the patch straight into registers (uniform loads)
  if constexpr (FB == 1) {
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
      for (int j = 0; j < 3; ++j) x1[a][j] = in_at(a, j);
  } else {
    if (c < 3 * NJ) xs[c / NJ][c % NJ] = in_at(c / NJ, c % NJ);
  }
  float wc[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) wc[k] = w[c * 9 + k];
  const float bc = bias[c];
  if constexpr (FB > 1) __syncthreads();
  float* ob = out + (size_t)b * out_bstride + ((size_t)o * 64 + f0) * 256 + c;
#pragma unroll 4
  for (int i = 0; i < FB; ++i) {
    const int f = f0 + i;
    float acc = bc;
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const int r = r0 + a, col = 2 * f - 1 + q;
        const bool live = r >= 0 && r < T && col >= 0 && col < 128;
        const float xv = FB == 1 ? x1[a][q] : xs[a][2 * i + q];
        acc += live ? wc[a * 3 + q] * xv : 0.f;
      }
    ob[(size_t)i * 256] = fmaxf(acc, 0.f);
  }
}

void conv0(const float* mel, long long mel_bstride, int mel_base, int T, float* out,
           long long out_bstride, int o_base, int n_out, int B, const float* w, const float* b,
           hipStream_t s) {
  if (n_out <= 0) return;
  if ((long long)n_out * (64 / 16) * B >= 1024)
    hipLaunchKernelGGL(conv0_kernel<16>, dim3(n_out * (64 / 16), B), dim3(256), 0, s, mel,
                       mel_bstride, mel_base, T, out, out_bstride, o_base, w, b);
  else
    hipLaunchKernelGGL(conv0_kernel<1>, dim3(n_out * 64, B), dim3(256), 0, s, mel, mel_bstride,
                       mel_base, T, out, out_bstride, o_base, w, b);
}

// Depthwise 3x3 stride 2: one workgroup = DW_FB output frequencies of one
// output row of one stream, thread = channel (its 3 x (2 DW_FB + 1) inputs and
// 9 weights in registers); DW_FB = 4 for large batches, 1 otherwise.
template <typename T, int DW_FB>
__global__ __launch_bounds__(256) void dw2d_kernel(const float* in, long long in_bstride,
                                                   int in_base, int len_in, int f_in, T* out,
                                                   long long out_bstride, int o_base,
                                                   const float* w, const float* bias) {
  constexpr int NJ = 2 * DW_FB + 1;
  const int f_out = (f_in + 1) / 2, nfb = (f_out + DW_FB - 1) / DW_FB;
  const int o = blockIdx.x / nfb, f0 = (blockIdx.x % nfb) * DW_FB, b = blockIdx.y, c = threadIdx.x;
  const float* ib = in + (size_t)b * in_bstride;
  const int r0 = 2 * (o_base + o) - 1;
  const int rlo = max(r0, max(0, in_base)), rhi = min(r0 + 2, len_in - 1);
  float x[3][NJ];
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = min(max(r0 + a, rlo), rhi), col = min(max(2 * f0 - 1 + j, 0), f_in - 1);
      x[a][j] = ib[((size_t)(r - in_base) * f_in + col) * 256 + c];
    }
  float wc[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) wc[k] = w[c * 9 + k];
  const float bc = bias[c];
#pragma unroll
  for (int i = 0; i < DW_FB; ++i) {
    const int f = f0 + i;
    if (f >= f_out) break;
    float acc = bc;
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const int r = r0 + a, col = 2 * f - 1 + q;
        const bool live = r >= 0 && r < len_in && col >= 0 && col < f_in;
        acc += live ? wc[a * 3 + q] * x[a][2 * i + q] : 0.f;
      }
    out[(size_t)b * out_bstride + ((size_t)o * f_out + f) * 256 + c] = from_f<T>(acc);
  }
}

void dw2d(const float* in, long long in_bstride, int in_base, int len_in, int f_in, void* out,
          long long out_bstride, int o_base, int n_out, int B, const float* w, const float* b,
          bool bf16, hipStream_t s) {
  if (n_out <= 0) return;
  const int f_out = (f_in + 1) / 2;
  const bool wide = (long long)n_out * ((f_out + 3) / 4) * B >= 1024;
  dim3 grid(n_out * (wide ? (f_out + 3) / 4 : f_out), B);
  if (bf16) {
    bf16_t* o = static_cast<bf16_t*>(out);
    if (wide)
      hipLaunchKernelGGL((dw2d_kernel<bf16_t, 4>), grid, dim3(256), 0, s, in, in_bstride, in_base,
                         len_in, f_in, o, out_bstride, o_base, w, b);
    else
      hipLaunchKernelGGL((dw2d_kernel<bf16_t, 1>), grid, dim3(256), 0, s, in, in_bstride, in_base,
                         len_in, f_in, o, out_bstride, o_base, w, b);
  } else {
    float* o = static_cast<float*>(out);
    if (wide)
      hipLaunchKernelGGL((dw2d_kernel<float, 4>), grid, dim3(256), 0, s, in, in_bstride, in_base,
                         len_in, f_in, o, out_bstride, o_base, w, b);
    else
      hipLaunchKernelGGL((dw2d_kernel<float, 1>), grid, dim3(256), 0, s, in, in_bstride, in_base,
                         len_in, f_in, o, out_bstride, o_base, w, b);
  }
}

// 8x frame stacking: out[b*n + j][r*128 + m] = mel[8(e0+j)+r][m], zero past T.
template <typename OT>
__global__ __launch_bounds__(256) void stack8_kernel(const float* mel, long long mel_bstride,
                                                     int mel_base, int T, int e0, int n, OT* out) {
  const int j = blockIdx.x, b = blockIdx.y;
  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = threadIdx.x + 256 * q, r = i >> 7, m = i & 127;
    const int t = min(8 * (e0 + j) + r, T - 1);
    v[q] = mel[(size_t)b * mel_bstride + (size_t)(t - mel_base) * 128 + m];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = threadIdx.x + 256 * q, r = i >> 7;
    out[((size_t)b * n + j) * 1024 + i] = from_f<OT>(8 * (e0 + j) + r < T ? v[q] : 0.f);
  }
}

void stack8(const float* mel, long long mel_bstride, int mel_base, int T, int e0, int n, int B,
            void* out, bool bf16, hipStream_t s) {
  if (n <= 0) return;
  if (bf16)
    hipLaunchKernelGGL((stack8_kernel<bf16_t>), dim3(n, B), dim3(256), 0, s, mel, mel_bstride,
                       mel_base, T, e0, n, static_cast<bf16_t*>(out));
  else
    hipLaunchKernelGGL((stack8_kernel<float>), dim3(n, B), dim3(256), 0, s, mel, mel_bstride,
                       mel_base, T, e0, n, static_cast<float*>(out));
}

// --------------------------------------------------------------- heads
// Sortformer head, fp32: sigmoid(W2 relu(W1 x + b1) + b2). One workgroup =
// 16 rows, 8 waves: the 192x192 layer runs on fp32 MFMA, wave w computing
// output columns 48(w%4).. +47 over half of K (w/4), the two halves summed in
// LDS. W1 is stored fragment by fragment (fragment (ks, ct) = lanes' values
// W1[16ct + l%16][4ks + l/16], 256 contiguous bytes), so each wave issues its
// 72 weight loads at once, in flight with the x rows and W2 (staged in LDS).
// The 192->S layer (S <= 8) gives each row 16 lanes (a DPP reduction), then
// the sigmoid.
__global__ __launch_bounds__(512) void head_sf_kernel(const float* x, int M, const float* w1f,
                                                      const float* b1, const float* w2,
                                                      const float* b2, int S, float* probs) {
  __shared__ float xs[16][196], hs[16][196], w2s[8][192];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r0 = blockIdx.x * 16;
  const int c16 = lane & 15, kq = lane >> 4, wc = w & 3, kh = w >> 2;
  for (int i = tid; i < S * 192; i += 512) w2s[i / 192][i % 192] = w2[i];
  float4 v[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {  // 16 rows x 48 float4
    const int i = min(tid + 512 * q, 767), r = i / 48, c = (i % 48) * 4;
    v[q] = *reinterpret_cast<const float4*>(x + (size_t)min(r0 + r, M - 1) * 192 + c);
  }
  float wf[24][3];
#pragma unroll
  for (int ks = 0; ks < 24; ++ks)
#pragma unroll
    for (int j = 0; j < 3; ++j)
      wf[ks][j] = w1f[(size_t)((24 * kh + ks) * 12 + 3 * wc + j) * 64 + lane];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = tid + 512 * q, r = i / 48, c = (i % 48) * 4;
    if (i < 768) {
      const bool live = r0 + r < M;
      xs[r][c] = live ? v[q].x : 0.f;
      xs[r][c + 1] = live ? v[q].y : 0.f;
      xs[r][c + 2] = live ? v[q].z : 0.f;
      xs[r][c + 3] = live ? v[q].w : 0.f;
    }
  }
  __syncthreads();
  f32x4 acc[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 24; ++ks) {
    const float av = xs[c16][4 * (24 * kh + ks) + kq];
#pragma unroll
    for (int j = 0; j < 3; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, wf[ks][j], acc[j], 0, 0, 0);
  }
  if (kh == 1) {  // upper K half: partial sums to LDS
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) hs[4 * kq + i][48 * wc + 16 * j + c16] = acc[j][i];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int n = 48 * wc + 16 * j + c16;
      const float bn = b1[n];
#pragma unroll
      for (int i = 0; i < 4; ++i) hs[4 * kq + i][n] = fmaxf(acc[j][i] + hs[4 * kq + i][n] + bn, 0.f);
    }
  }
  __syncthreads();
  if (tid < 256) {
    const int r = tid >> 4, sub = tid & 15;  // 16 lanes per row
    for (int sp = 0; sp < S; ++sp) {
      float z = 0.f;
#pragma unroll
      for (int k = sub; k < 192; k += 16) z += hs[r][k] * w2s[sp][k];
      z = row16_sum(z);
      if (sub == 0 && r0 + r < M)
        probs[(size_t)(r0 + r) * S + sp] = 1.0f / (1.0f + expf(-(z + b2[sp])));
    }
  }
}

void head_sortformer(const float* x, int M, const float* w1f, const float* b1, const float* w2,
                     const float* b2, int S, float* probs, hipStream_t s) {
  if (M <= 0 || S < 1 || S > 8) return;
  hipLaunchKernelGGL(head_sf_kernel, dim3((M + 15) / 16), dim3(512), 0, s, x, M, w1f, b1, w2, b2, S,
                     probs);
}

// Nemotron head, fp32: z = Wh x + bh (80 ms logits), p80 = sigmoid(z);
// ConvTranspose1d(8,8,k=8,s=8): p10[8t+r][o] = sigmoid(ub[o] + sum_i z[i] uw[i][o][r]).
__global__ __launch_bounds__(256) void head_nm_kernel(const float* x, int M, const float* hw,
                                                      const float* hb, const float* uw,
                                                      const float* ub, float* p80, float* p10) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;
  float xv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) xv[i] = x[(size_t)row * 512 + lane + 64 * i];
  float z[8];
#pragma unroll
  for (int sp = 0; sp < 8; ++sp) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a += xv[i] * hw[sp * 512 + lane + 64 * i];
    z[sp] = wave_sum(a) + hb[sp];
  }
  if (lane < 8) p80[(size_t)row * 8 + lane] = 1.0f / (1.0f + expf(-z[lane & 7]));
  const int r = lane >> 3, o = lane & 7;
  float v = ub[o];
#pragma unroll
  for (int i = 0; i < 8; ++i) v += z[i] * uw[(i * 8 + o) * 8 + r];
  p10[((size_t)row * 8 + r) * 8 + o] = 1.0f / (1.0f + expf(-v));
}

void head_nemotron(const float* x, int M, const float* hw, const float* hb, const float* uw,
                   const float* ub, float* p80, float* p10, hipStream_t s) {
  if (M <= 0) return;
  hipLaunchKernelGGL(head_nm_kernel, dim3((M + 3) / 4), dim3(256), 0, s, x, M, hw, hb, uw, ub,
                     p80, p10);
}

// ------------------------------------------------------- state plumbing
__global__ void copy_rows_kernel(const float* src, long long sb, int sl, float* dst, long long db,
                                 int dl, int cols) {
  const int r = blockIdx.x, b = blockIdx.y;
  const float* sp = src + (size_t)b * sb + (size_t)r * sl;
  float* dp = dst + (size_t)b * db + (size_t)r * dl;
  for (int c = threadIdx.x; c < cols; c += blockDim.x) dp[c] = sp[c];
}

void copy_rows(const float* src, long long sb, int sl, float* dst, long long db, int dl, int B,
               int rows, int cols, hipStream_t s) {
  if (rows <= 0 || B <= 0) return;
  hipLaunchKernelGGL(copy_rows_kernel, dim3(rows, B), dim3(cols >= 256 ? 256 : 64), 0, s, src, sb,
                     sl, dst, db, dl, cols);
}

__global__ void copy_rows_nv_kernel(const float* src, long long sb, int sl, float* dst,
                                    long long db, int dl, int cols, const int* nv) {
  const int r = blockIdx.x, b = blockIdx.y;
  const bool live = r < *nv;
  const float* sp = src + (size_t)b * sb + (size_t)r * sl;
  float* dp = dst + (size_t)b * db + (size_t)r * dl;
  for (int c = threadIdx.x; c < cols; c += blockDim.x) dp[c] = live ? sp[c] : 0.f;
}

void copy_rows_nv(const float* src, long long sb, int sl, float* dst, long long db, int dl, int B,
                  int rows, int cols, const int* nv, hipStream_t s) {
  if (rows <= 0 || B <= 0) return;
  hipLaunchKernelGGL(copy_rows_nv_kernel, dim3(rows, B), dim3(cols >= 256 ? 256 : 64), 0, s, src,
                     sb, sl, dst, db, dl, cols, nv);
}

__global__ void widen_kernel(const void* src, bool bf, float* dst, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n)
    dst[i] = bf ? bf2f(static_cast<const bf16_t*>(src)[i]) : static_cast<const float*>(src)[i];
}

void widen(const void* src, bool src_bf16, float* dst, long long n, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(widen_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src,
                     src_bf16, dst, n);
}

__global__ void pool_rows_kernel(const float* src, long long s_bstride, float* dst,
                                 long long d_bstride, int n_out, int r, int cols) {
  const int i = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
  if (i >= n_out * cols) return;
  const int k = i / cols, c = i % cols;
  const float* p = src + (size_t)b * s_bstride + (size_t)k * r * cols + c;
  float acc = 0.f;
  for (int q = 0; q < r; ++q) acc += p[(size_t)q * cols];
  dst[(size_t)b * d_bstride + (size_t)k * cols + c] = acc / (float)r;
}

void pool_rows(const float* src, long long s_bstride, float* dst, long long d_bstride, int B,
               int n_out, int r, int cols, hipStream_t s) {
  if (n_out <= 0 || B <= 0) return;
  hipLaunchKernelGGL(pool_rows_kernel, dim3((n_out * cols + 255) / 256, B), dim3(256), 0, s, src,
                     s_bstride, dst, d_bstride, n_out, r, cols);
}

__global__ void ring_write_kernel(const float* src, long long src_bstride, long long n,
                                  float* ring, long long cap, long long start) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (i < n) ring[(size_t)b * cap + ((start + i) & (cap - 1))] = src[(size_t)b * src_bstride + i];
}

void ring_write(const float* src, long long src_bstride, long long n, int B, float* ring,
                long long cap, long long start, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(ring_write_kernel, dim3((unsigned)((n + 255) / 256), B), dim3(256), 0, s, src,
                     src_bstride, n, ring, cap, start);
}

__global__ void fill_i32_kernel(int* p, long long n, int v) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void fill_f64_kernel(double* p, long long n, double v) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}
void fill_i32(int* p, long long n, int v, hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
}
void fill_f64(double* p, long long n, double v, hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(fill_f64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
}

// FIFO prediction refresh and chunk append: state rows [Lc, Lc+nrows) take
// the window's probabilities at the same rows and are marked real frames.
__global__ void refresh_kernel(const float* wp, int W, int S, int Lc, int nrows, float* P, int* ph,
                               int cap) {
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < nrows * S; i += blockDim.x) {
    const int r = Lc + i / S, sp = i % S;
    P[((size_t)b * cap + r) * S + sp] = wp[((size_t)b * W + r) * S + sp];
  }
  for (int i = threadIdx.x; i < nrows; i += blockDim.x) ph[(size_t)b * cap + Lc + i] = 0;
}

void refresh_probs(const float* wp, int W, int S, int B, int Lc, int nrows, float* P, int* ph,
                   int cap, hipStream_t s) {
  if (nrows <= 0) return;
  hipLaunchKernelGGL(refresh_kernel, dim3(B), dim3(256), 0, s, wp, W, S, Lc, nrows, P, ph, cap);
}

// Silence statistics of the frames popped from the FIFO: rows [r0, r0+n) in
// order; a frame whose largest probability is <= 0.5 adds its embedding to
// the float64 running sum (one thread per dimension, so the additions happen
// in frame order) and increments the count.
__global__ __launch_bounds__(512) void silence_kernel(const float* E, const float* P, int cap, int D,
                                                      int S, int r0, int n, double* sum, int* cnt) {
  __shared__ unsigned char silent[1024];
  const int b = blockIdx.x;
  const float* Eb = E + (size_t)b * cap * D;
  const float* Pb = P + (size_t)b * cap * S;
  for (int r = threadIdx.x; r < n; r += blockDim.x) {
    float mx = Pb[(size_t)(r0 + r) * S];
    for (int sp = 1; sp < S; ++sp) mx = fmaxf(mx, Pb[(size_t)(r0 + r) * S + sp]);
    silent[r] = mx <= 0.5f;
  }
  __syncthreads();
  int added = 0;
  for (int r = 0; r < n; ++r) added += silent[r];
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    double acc = sum[(size_t)b * D + d];
    int r = 0;
    for (; r + 8 <= n; r += 8) {  // eight loads in flight, added in frame order
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = Eb[(size_t)(r0 + r + q) * D + d];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc = silent[r + q] ? acc + (double)v[q] : acc;
    }
    for (; r < n; ++r) {
      const float v = Eb[(size_t)(r0 + r) * D + d];
      acc = silent[r] ? acc + (double)v : acc;
    }
    sum[(size_t)b * D + d] = acc;
  }
  if (threadIdx.x == 0) cnt[b] += added;
}

void silence_update(const float* E, const float* P, int cap, int D, int S, int B, int r0, int n,
                    double* sum, int* cnt, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(silence_kernel, dim3(B), dim3(512), 0, s, E, P, cap, D, S, r0, n, sum, cnt);
}

}  // namespace sf
