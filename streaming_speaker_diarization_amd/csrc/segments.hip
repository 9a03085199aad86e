// Speaker-activity probabilities -> speech segments (model card, Output;
// NeMo diarize() Returns; Transformers extract_speaker_dict). One wave per
// (stream, speaker) track walks the frames 64 at a time (the loads of 16
// chunks issued together): the hysteresis
// state of every frame is the on/off decision of the last decisive frame at
// or before it (p > onset or p <= offset), found from two ballots, so a
// chunk is resolved without a serial pass; the run boundaries are then
// visited in time order (wave-uniform) to pad, merge and filter. Built with
// floating-point contraction off: the fp64 times are plain IEEE products and
// sums.
#include "sortformer.h"
#include "kernels.h"

namespace sf {

struct SegState {
  double ps, pe;  // pending segment
  bool have;
  long long n;    // segments found (written while below the capacity, which the
                  // host sizes for the most a track can hold)
  long long cap;
};

__device__ __forceinline__ void seg_emit(SegState& st, double min_on, sf_segment* out, int spk,
                                         int b, bool writer) {
  if (st.have && st.pe - st.ps >= min_on) {
    if (writer && st.n < st.cap) {
      sf_segment sg;
      sg.start_s = st.ps;
      sg.end_s = st.pe;
      sg.speaker = spk;
      sg.stream = b;
      out[st.n] = sg;
    }
    ++st.n;
  }
}

__device__ __forceinline__ void seg_run(SegState& st, int f0, int f1, double dt, double total,
                                        const sf_segment_params& p, sf_segment* out, int spk, int b,
                                        bool writer) {
  const double s0 = (double)f0 * dt - p.pad_onset, e0 = (double)f1 * dt + p.pad_offset;
  const double s = s0 > 0.0 ? s0 : 0.0;
  const double e = e0 < total ? e0 : total;
  if (st.have && s - st.pe < p.min_duration_off) {
    st.pe = e > st.pe ? e : st.pe;
    return;
  }
  seg_emit(st, p.min_duration_on, out, spk, b, writer);
  st.ps = s;
  st.pe = e;
  st.have = true;
}

__global__ __launch_bounds__(64) void segments_kernel(const float* probs, int T, int S, double dt,
                                                      sf_segment_params prm, sf_segment* out,
                                                      long long cap, long long* counts) {
  const int track = blockIdx.x, b = track / S, spk = track % S, lane = threadIdx.x;
  const float* p = probs + (size_t)b * T * S + spk;
  sf_segment* o = out + (size_t)track * cap;
  const double total = (double)T * dt;
  const unsigned long long le = lane == 63 ? ~0ull : ((1ull << (lane + 1)) - 1ull);
  SegState st{0.0, 0.0, false, 0, cap};
  unsigned long long carry = 0;  // state of the frame before this chunk
  int run0 = 0;                  // start frame of the open run
  constexpr int U = 16;  // chunks whose loads are issued together
  for (int cb = 0; cb < T; cb += 64 * U) {
    float vu[U];
#pragma unroll
    for (int u = 0; u < U; ++u) vu[u] = p[(size_t)min(cb + 64 * u + lane, T - 1) * S];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c0 = cb + 64 * u;
      if (c0 >= T) break;
      const int t = c0 + lane;
      const float v = vu[u];
      const bool live = t < T;
      const bool on = live && v > prm.onset;
      const bool decisive = !live || on || v <= prm.offset;  // past the end counts as off
      const unsigned long long D = __ballot(decisive), O = __ballot(on);
      const unsigned long long dm = D & le;
      const int state = dm ? (int)((O >> (63 - __clzll(dm))) & 1ull) : (int)carry;
      const unsigned long long Sm = __ballot(state);
      const unsigned long long prev = (Sm << 1) | carry;
      unsigned long long ev = (Sm & ~prev) | (~Sm & prev);  // starts and ends
      carry = Sm >> 63;
      while (ev) {
        const int q = __ffsll((long long)ev) - 1;
        ev &= ev - 1;
        if ((Sm >> q) & 1ull) {
          run0 = c0 + q;
        } else {
          seg_run(st, run0, c0 + q, dt, total, prm, o, spk, b, lane == 0);
        }
      }
    }
  }
  if (carry) seg_run(st, run0, T, dt, total, prm, o, spk, b, lane == 0);
  seg_emit(st, prm.min_duration_on, o, spk, b, lane == 0);
  if (lane == 0) counts[track] = st.n;
}

void segments(const float* probs, int B, int T, int S, double dt, const sf_segment_params& prm,
              sf_segment* out, long long cap, long long* counts, hipStream_t s) {
  hipLaunchKernelGGL(segments_kernel, dim3(B * S), dim3(64), 0, s, probs, T, S, dt, prm, out, cap,
                     counts);
}

}  // namespace sf
