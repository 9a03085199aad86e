// Speaker-cache compression ("Streaming Sortformer Diarizer" card, Streaming
// Architecture: on overflow keep the highest log-odds-scored frames per
// speaker plus silence placeholders). One workgroup per stream.
//
// Score: the log-odds score log p_s - log(1-p_s) + sum_{j!=s} log(1-p_j) is
// ranked through the monotone-equivalent key
//   K_s = (p_s/(1-p_s)) * prod_{j!=s, ascending} (1-p_j),  p clamped to [2^-24, 1-2^-24],
// computed with correctly rounded float64 divide/multiply only (1-p is exact
// for fp32 p), so the ranking is reproducible bit for bit on any IEEE host.
// Frames with p_s > 0.5 that are not placeholders are eligible for speaker s;
// the k largest keys win, ties going to the earlier frame. Block s of the new
// cache (floor(C/S) slots) holds the winners in time order, then
// placeholders; trailing slots are placeholders. A placeholder carries the
// running silence mean (float64 sum / count, rounded to fp32; zero before any
// silence) and zero probabilities. The rows after the old cache (FIFO and
// look-ahead) move up behind the new cache. Selection runs in one workgroup
// per stream; the row copies are spread over one workgroup per row.
// This file is built with floating-point contraction disabled.
#include "kernels.h"

namespace sf {

#define CMP_MAXM 1024
#define CMP_MAXS 8
// candidates (cache + popped frames) and cache slots never exceed the state's
// capacity, which the ABI bounds by the largest window
static_assert(CMP_MAXM >= SF_MAX_WINDOW, "compression arrays must hold a full window");

__global__ __launch_bounds__(512) void compress_kernel(const float* E, const float* P,
                                                       const int* ph, int cap, int D, int S,
                                                       int M, int tail, const double* sil_sum,
                                                       const int* sil_cnt, int C, int per, int k,
                                                       int* slots) {
  __shared__ double keys[CMP_MAXM * CMP_MAXS];   // -1 marks an ineligible (frame, speaker)
  __shared__ int slot_src[CMP_MAXM];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* Eb = E + (size_t)b * cap * D;
  const float* Pb = P + (size_t)b * cap * S;
  const int* phb = ph + (size_t)b * cap;

  for (int idx = tid; idx < M * S; idx += blockDim.x) {
    const int m = idx / S, s = idx % S;
    const float ps = Pb[(size_t)m * S + s];
    double key = -1.0;
    if (ps > 0.5f && phb[m] == 0) {
      const double lo = 5.9604644775390625e-8, hi = 1.0 - 5.9604644775390625e-8;
      double pc = fmin(fmax((double)ps, lo), hi);
      double kk = pc / (1.0 - pc);
      for (int j = 0; j < S; ++j) {
        if (j == s) continue;
        const double pj = fmin(fmax((double)Pb[(size_t)m * S + j], lo), hi);
        kk = kk * (1.0 - pj);
      }
      key = kk;
    }
    keys[idx] = key;
  }
  __syncthreads();
  // Selection: rank among eligible frames of the same speaker.
  __shared__ unsigned char sel[CMP_MAXM * CMP_MAXS];
  for (int idx = tid; idx < M * S; idx += blockDim.x) {
    const int m = idx / S, s = idx % S;
    const double key = keys[idx];
    unsigned char chosen = 0;
    if (key > 0.0) {
      int rank = 0;
      for (int q = 0; q < M && rank < k; ++q) {
        const double kq = keys[q * S + s];
        rank += (kq > key) || (kq == key && q < m);
      }
      chosen = rank < k;
    }
    sel[idx] = chosen;
  }
  __syncthreads();
  // Slot assignment: wave s compacts speaker s's winners in frame order.
  for (int s = wave; s < S; s += blockDim.x / 64) {
    int base = 0;
    for (int m0 = 0; m0 < M; m0 += 64) {
      const int m = m0 + lane;
      const bool f = m < M && sel[m * S + s];
      const unsigned long long mask = __ballot(f);
      const int pos = base + __popcll(mask & ((1ull << lane) - 1ull));
      if (f) slot_src[s * per + pos] = m;
      base += __popcll(mask);
    }
    for (int r = base + lane; r < per; r += 64) slot_src[s * per + r] = -1;
  }
  for (int r = S * per + tid; r < C; r += blockDim.x) slot_src[r] = -1;
  __syncthreads();

  // slot map for the gather: >= 0 source frame, -1 placeholder
  for (int r = tid; r < C; r += blockDim.x) slots[(size_t)b * cap + r] = slot_src[r];
}

// Builds the new cache (one workgroup per row): slot rows take their source
// frame or the placeholder (silence mean, zero probabilities); the FIFO and
// look-ahead rows that followed the old cache move up behind it.
__global__ __launch_bounds__(128) void cache_gather_kernel(const float* E, const float* P,
                                                           const int* ph, int cap, int D, int S,
                                                           int M, int C, const int* slots,
                                                           const double* sil_sum,
                                                           const int* sil_cnt, float* E2, float* P2,
                                                           int* ph2) {
  const int r = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int src = r < C ? slots[(size_t)b * cap + r] : M + (r - C);
  const float* Eb = E + (size_t)b * cap * D;
  float* E2r = E2 + ((size_t)b * cap + r) * D;
  if (src >= 0) {
    for (int d = 4 * t; d < D; d += 512)
      *reinterpret_cast<float4*>(E2r + d) = *reinterpret_cast<const float4*>(Eb + (size_t)src * D + d);
  } else {
    const int cnt = sil_cnt[b];
    for (int d = t; d < D; d += 128)
      E2r[d] = cnt > 0 ? (float)(sil_sum[(size_t)b * D + d] / (double)cnt) : 0.f;
  }
  if (t < S) P2[((size_t)b * cap + r) * S + t] = src >= 0 ? P[((size_t)b * cap + src) * S + t] : 0.f;
  if (t == 0) ph2[(size_t)b * cap + r] = src >= 0 ? (r < C ? 0 : ph[(size_t)b * cap + src]) : 1;
}

void compress_cache(const float* E, const float* P, const int* ph, int cap, int D, int S, int B,
                    int M, int tail, const double* sil_sum, const int* sil_cnt, int C, int per,
                    int k, float* E2, float* P2, int* ph2, int* slots, hipStream_t s) {
  klaunch(PROF_CACHE, 0.0, (double)B * M * (S + 1) * 4, compress_kernel, dim3(B), dim3(512), s, E,
          P, ph, cap, D, S, M, tail, sil_sum, sil_cnt, C, per, k, slots);
  klaunch(PROF_CACHE, 0.0, (double)B * (C + tail) * (D + S + 1) * 8, cache_gather_kernel,
          dim3(C + tail, B), dim3(128), s, E, P, ph, cap, D, S, M, C, (const int*)slots, sil_sum,
          sil_cnt, E2, P2, ph2);
}

}  // namespace sf
