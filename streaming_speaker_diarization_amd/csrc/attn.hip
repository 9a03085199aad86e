// Multi-head self-attention over one encoder window, flash-style.
//
// One workgroup = 16 query rows of one (stream, head); its four waves take
// the 64-frame key tiles round-robin (so a window of a few hundred frames
// still spreads over many waves) and merge their online-softmax states at the
// end. MFMA B operands (K rows, the relative-position band, V transposed per
// head by the QKV projection) are read straight from global memory/L2 into
// registers, the next tile's K and band while the current one is computed;
// LDS only carries the score shift and the re-layout of P for P.V. Running
// max/sum in fp32 in the exp2 domain; row reductions with DPP.
//
// Modes:
//  ATT_RELPOS  FastConformer relative-position attention ("Streaming
//    Sortformer Diarizer" card, torch.export Fixes 6: rel_shift). The score of
//    query i and key j is [(q_i+u).k_j + (q_i+v).p(i-j)]/sqrt(d). The
//    projections p(delta) are input-independent and precomputed for every
//    delta; per key tile the 80-row band of p that the tile's (i, j) pairs
//    touch feeds one more MFMA product G = (q+v).band^T, and the shift is done
//    by indexing G (through LDS) at column i-j+63 — no padded score matrix is
//    materialised.
//  ATT_ROPE    rotary embedding on q and k (rotate-half, positions = window
//    index, which restart at every chunk) for the Nemotron-style layers.
//  ATT_PLAIN   standard scaled dot-product attention (transformer, d=24,
//    zero-padded to 32 for the MFMA K dimension).
// Keys at index >= n_valid are right padding and are masked.
#include "kernels.h"

namespace sf {

template <typename T> struct Pack;
template <> struct Pack<float> {
  __device__ static float make(const float* v) { return v[0]; }
};
template <> struct Pack<bf16_t> {
  __device__ static bf16x8_t make(const float* v) { return pack_bf16x8(v); }
};

// Fragment I/O: EPF consecutive elements (8 bf16 or 1 fp32) as one load.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
  typedef bf16x8_t type;
  __device__ static type load(const bf16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }
  __device__ static float get(const type& f, int e) {
    return bf2f(__builtin_bit_cast(u16x8, f)[e]);
  }
  __device__ static type zero_if(const type& f, unsigned live_mask) {
    u16x8 u = __builtin_bit_cast(u16x8, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = (live_mask >> e) & 1u ? u[e] : (uint16_t)0;
    return __builtin_bit_cast(bf16x8_t, u);
  }
};
template <> struct Frag<float> {
  typedef float type;
  __device__ static type load(const float* p) { return *p; }
  __device__ static float get(const type& f, int) { return f; }
  __device__ static type zero_if(const type& f, unsigned live_mask) { return live_mask & 1u ? f : 0.f; }
};

// LDS hand-off between lanes of one wave (the producer and consumer are the
// same wave, so waiting for its LDS operations is enough).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt/expcnt unconstrained
  __builtin_amdgcn_wave_barrier();
}

// One workgroup = 16 query rows of one (stream, head); its NW waves take the
// key tiles (64 frames) round-robin and merge their partial softmax states at
// the end. MFMA B operands are read straight from global memory (L2):
//  K rows   [key][dim]          -> scores  S = Q K^T
//  p band   [delta][dim]        -> G = (q+v) p(delta)^T  (relative position)
//  V^T rows [dim][key]          -> O += P V
// so the only LDS traffic is the score shift (G) and the re-layout of P.
template <typename T, int HD, int MODE, int NW>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnArgs a) {
  using M_ = MF<T>;
  using F = Frag<T>;
  typedef typename F::type frag_t;
  constexpr int KI = M_::KI;
  constexpr int EPF = KI / 4;              // consecutive elements per fragment
  constexpr int HDP = HD <= 32 ? 32 : 64;  // head dim padded for MFMA
  constexpr int NQF = HDP / KI;            // k-steps over head dims
  constexpr int NKF = 64 / KI;             // k-steps over a 64-key tile
  constexpr int NDT = HDP / 16;            // output column tiles
  constexpr int LDP = 64 + 16 / (int)sizeof(T);
  constexpr bool REL = MODE == ATT_RELPOS;
  constexpr bool ROPE = MODE == ATT_ROPE;
  static_assert(!ROPE || HD == 64, "rotary layers use 64-dim heads");
  __shared__ float Gs[REL ? NW * 16 * 81 : 1];
  __shared__ __align__(16) T Ps[NW * 16 * LDP];
  __shared__ float Ms[NW][16], Ls[NW][16];
  __shared__ float Os[NW][16][HDP + 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int iq0 = blockIdx.x * 16, h = blockIdx.y, b = blockIdx.z;
  const T* qkv = static_cast<const T*>(a.qkv);
  const size_t rowbase = (size_t)b * a.W;
  const float sl2 = a.scale * 1.4426950408889634f;
  const T* vtb = static_cast<const T*>(a.vt) + (size_t)(b * a.H + h) * HD * a.vpitch;

  // ---- query fragments for row iq0+c16 (element e of fragment ks is dim
  // ks*KI + EPF*g + e)
  frag_t qa[NQF], qb[NQF];
  {
    const int qi = iq0 + c16, qc = min(qi, a.W - 1);
    float q[NQF][EPF];
#pragma unroll
    for (int ks = 0; ks < NQF; ++ks)
#pragma unroll
      for (int e = 0; e < EPF; ++e) {
        const int d = ks * KI + EPF * g + e;
        q[ks][e] = to_f<T>(qkv[(rowbase + qc) * a.ldq + a.qoff + h * HD + min(d, HD - 1)]);
      }
#pragma unroll
    for (int ks = 0; ks < NQF; ++ks)
#pragma unroll
      for (int e = 0; e < EPF; ++e) {
        const int d = ks * KI + EPF * g + e;
        q[ks][e] = (qi < a.W && d < HD) ? q[ks][e] : 0.f;
      }
    if constexpr (ROPE) {
      constexpr int HALF = 32 / KI;  // fragment offset of dim d+32
#pragma unroll
      for (int ks = 0; ks < HALF; ++ks)
#pragma unroll
        for (int e = 0; e < EPF; ++e) {
          const int d = ks * KI + EPF * g + e;
          const float c = a.rope[(qc * 32 + d) * 2], s = a.rope[(qc * 32 + d) * 2 + 1];
          const float x1 = q[ks][e], x2 = q[ks + HALF][e];
          q[ks][e] = x1 * c - x2 * s;
          q[ks + HALF][e] = x2 * c + x1 * s;
        }
    }
#pragma unroll
    for (int ks = 0; ks < NQF; ++ks) {
      float ua[EPF], va[EPF];
#pragma unroll
      for (int e = 0; e < EPF; ++e) {
        const int d = ks * KI + EPF * g + e;
        ua[e] = q[ks][e];
        va[e] = q[ks][e];
        if constexpr (REL) {
          const float ub = a.ub[h * HD + min(d, HD - 1)], vb = a.vb[h * HD + min(d, HD - 1)];
          ua[e] += d < HD ? ub : 0.f;
          va[e] += d < HD ? vb : 0.f;
        }
      }
      qa[ks] = Pack<T>::make(ua);
      qb[ks] = Pack<T>::make(va);
    }
  }
  // live-dimension mask of this lane's fragment elements for each k-step
  auto dim_mask = [&](int ks) {
    unsigned m = 0;
#pragma unroll
    for (int e = 0; e < EPF; ++e) m |= (ks * KI + EPF * g + e < HD ? 1u : 0u) << e;
    return m;
  };

  frag_t kf[4][NQF], bfr[REL ? 5 : 1][NQF], vf[NDT][NKF];
  // K and position-band fragments of key tile j0 (issued together)
  auto load_kb = [&](int j0) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int j = min(j0 + 16 * nt + c16, a.W - 1);
      const T* kr = qkv + (rowbase + j) * a.ldq + a.koff + h * HD;
#pragma unroll
      for (int ks = 0; ks < NQF; ++ks) kf[nt][ks] = F::load(kr + min(ks * KI + EPF * g, HD - EPF));
    }
    if constexpr (REL) {
      const int dbase = iq0 - j0 - 63 + a.p_center;
#pragma unroll
      for (int ct = 0; ct < 5; ++ct) {
        const int tr = min(max(dbase + 16 * ct + c16, 0), 2 * a.p_center);
        const T* pr = static_cast<const T*>(a.P) + (size_t)tr * a.ldp + h * HD;
#pragma unroll
        for (int ks = 0; ks < NQF; ++ks) bfr[ct][ks] = F::load(pr + min(ks * KI + EPF * g, HD - EPF));
      }
    }
  };
  auto load_v = [&](int j0) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const T* vr = vtb + (size_t)min(16 * dt + c16, HD - 1) * a.vpitch;
#pragma unroll
      for (int ks = 0; ks < NKF; ++ks)
        vf[dt][ks] = F::load(vr + min(j0 + ks * KI + EPF * g, a.vpitch - EPF));
    }
  };

  f32x4 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { mrow[r] = -INFINITY; lrow[r] = 0.f; }

  const int n_valid = a.nv ? *a.nv : a.n_valid;
  const int ntile = (n_valid + 63) / 64;
  if (w < ntile) load_kb(w * 64);
  for (int kt = w; kt < ntile; kt += NW) {
    const int j0 = kt * 64;
    load_v(j0);
    // the loads are unconditional: zero what lies outside the head (head
    // dims not a multiple of the k-step) or the position table (a band
    // past either end: wave-uniform test)
    if constexpr (HD % KI != 0) {
#pragma unroll
      for (int ks = 0; ks < NQF; ++ks) {
        const unsigned dm = dim_mask(ks);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) kf[nt][ks] = F::zero_if(kf[nt][ks], dm);
      }
    }
    if constexpr (REL) {
      const int dbase = iq0 - j0 - 63;
      if (dbase < -a.p_center || dbase + 79 > a.p_center) {
#pragma unroll
        for (int ks = 0; ks < NQF; ++ks)
#pragma unroll
          for (int ct = 0; ct < 5; ++ct) {
            const int dl = dbase + 16 * ct + c16;
            bfr[ct][ks] =
                F::zero_if(bfr[ct][ks], (dl >= -a.p_center && dl <= a.p_center) ? dim_mask(ks) : 0u);
          }
      }
    }
    if constexpr (ROPE) {  // rotate the keys (positions = window index)
      constexpr int HALF = 32 / KI;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int pos = min(j0 + 16 * nt + c16, a.W - 1);
#pragma unroll
        for (int ks = 0; ks < HALF; ++ks) {
          float x1[EPF], x2[EPF];
#pragma unroll
          for (int e = 0; e < EPF; ++e) {
            const int d = ks * KI + EPF * g + e;
            const float c = a.rope[(pos * 32 + d) * 2], s = a.rope[(pos * 32 + d) * 2 + 1];
            const float k1 = F::get(kf[nt][ks], e), k2 = F::get(kf[nt][ks + HALF], e);
            x1[e] = k1 * c - k2 * s;
            x2[e] = k2 * c + k1 * s;
          }
          kf[nt][ks] = Pack<T>::make(x1);
          kf[nt][ks + HALF] = Pack<T>::make(x2);
        }
      }
    }
    // ---- scores
    f32x4 S[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      S[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NQF; ++ks) S[nt] = M_::mma(qa[ks], kf[nt][ks], S[nt]);
    }
    if constexpr (REL) {
      // G[i][c] = (q_i+v).p(delta_c), band row c <-> delta iq0-j0-63+c; the
      // score of (i, j) takes column i-j+63.
      float* G = &Gs[w * 16 * 81];
#pragma unroll
      for (int ct = 0; ct < 5; ++ct) {
        f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NQF; ++ks) acc = M_::mma(qb[ks], bfr[ct][ks], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) G[(4 * g + r) * 81 + 16 * ct + c16] = acc[r];
      }
      wave_lds_sync();
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[nt][r] += G[(4 * g + r) * 81 + (4 * g + r) - (16 * nt + c16) + 63];
    }
    if (kt + NW < ntile) load_kb(j0 + 64 * NW);  // next tile of this wave, in flight now

    // ---- online softmax (log2 domain: the running max is kept scaled by
    // scale*log2(e), p = 2^(s*scale*log2(e) - m)); keys past n_valid exist
    // only in the last tile
    if (j0 + 64 > n_valid) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[nt][r] = j0 + 16 * nt + c16 < n_valid ? S[nt][r] : -INFINITY;
    }
    float mx[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      mx[r] = fmaxf(fmaxf(S[0][r], S[1][r]), fmaxf(S[2][r], S[3][r]));
    T* Pw = &Ps[w * 16 * LDP];
    float alpha[4];
    bool moved = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mnew = fmaxf(mrow[r], row16_max(mx[r]) * sl2);
      alpha[r] = __builtin_amdgcn_exp2f(mrow[r] - mnew);
      moved |= mnew != mrow[r];
      float rs = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float p = __builtin_amdgcn_exp2f(fmaf(S[nt][r], sl2, -mnew));
        rs += p;
        Pw[(4 * g + r) * LDP + 16 * nt + c16] = from_f<T>(p);
      }
      lrow[r] = lrow[r] * alpha[r] + row16_sum(rs);
      mrow[r] = mnew;
    }
    if (__ballot(moved)) {  // rescale only when some row's max moved
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) O[dt][r] *= alpha[r];
    }
    // V^T columns past the window (last tile) or the head are zero
    if (j0 + 64 > a.W) {
#pragma unroll
      for (int ks = 0; ks < NKF; ++ks) {
        unsigned km = 0;
#pragma unroll
        for (int e = 0; e < EPF; ++e) km |= (j0 + ks * KI + EPF * g + e < a.W ? 1u : 0u) << e;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) vf[dt][ks] = F::zero_if(vf[dt][ks], km);
      }
    }
    if constexpr (HD % 16 != 0) {
#pragma unroll
      for (int ks = 0; ks < NKF; ++ks)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          vf[dt][ks] = F::zero_if(vf[dt][ks], 16 * dt + c16 < HD ? 0xFFu : 0u);
    }
    wave_lds_sync();
    // ---- O += P.V
#pragma unroll
    for (int ks = 0; ks < NKF; ++ks) {
      const auto pa = M_::ld(&Pw[c16 * LDP + ks * KI], lane);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) O[dt] = M_::mma(pa, vf[dt][ks], O[dt]);
    }
  }

  // Output projection fused (bf16 rel-pos and rotary layers): this wave's Wo fragments
  // (output columns 128w.., the head's 64 input columns), in flight during
  // the merge.
  constexpr bool FWO = (REL || ROPE) && sizeof(T) == 2 && HD == 64 && NW == 4;
  const bool fwo = FWO && a.wo_f != nullptr;
  bf16x8_t wof[FWO ? 8 : 1][2];
  if constexpr (FWO) {
    if (fwo) {
      const bf16_t* wo = static_cast<const bf16_t*>(a.wo_f);
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          wof[j][ks] = *reinterpret_cast<const bf16x8_t*>(
              wo + ((size_t)(8 * w + j) * 16 + 2 * h + ks) * 512 + 8 * lane);
    }
  }

  // ---- merge the four waves' partial softmax states
  if (c16 == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) { Ms[w][4 * g + r] = mrow[r]; Ls[w][4 * g + r] = lrow[r]; }
  }
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) Os[w][4 * g + r][16 * dt + c16] = O[dt][r];
  __syncthreads();
  T* ctx = static_cast<T*>(a.ctx);
  for (int o = tid; o < 16 * HD; o += NW * 64) {
    const int r = o / HD, d = o % HD, i = iq0 + r;
    float mx = Ms[0][r];
#pragma unroll
    for (int v = 1; v < NW; ++v) mx = fmaxf(mx, Ms[v][r]);
    float l = 0.f, acc = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float f = exp2f(Ms[v][r] - mx);  // waves without tiles: exp2(-inf) = 0
      l += Ls[v][r] * f;
      acc += Os[v][r][d] * f;
    }
    const T cv = from_f<T>(acc / l);
    if (i < a.W) ctx[(rowbase + i) * a.ldc + h * HD + d] = cv;
    if constexpr (FWO) Ps[r * 72 + d] = i < a.W ? cv : T(0);  // A operand of the projection
  }
  if constexpr (FWO) {
    if (fwo) {  // part[h][row] = ctx_h(row) . Wo[:, 64h..64h+63]^T, 128 columns per wave
      __syncthreads();
      bf16x8_t af[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) af[ks] = M_::ld(&Ps[c16 * 72 + ks * 32], lane);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc = M_::mma(af[ks], wof[j][ks], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = iq0 + 4 * g + r;
          if (i < a.W)
            a.part[((size_t)h * a.M + rowbase + i) * 512 + 128 * w + 16 * j + c16] = acc[r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Throughput form for batched windows (streams x window above 4096 rows),
// bf16: one workgroup = 128 query rows (32 per wave, as two 16-row sets) of
// one (stream, head). Each 64-key tile of K, V^T and (relative positions) the
// 192-row band of p(delta) its (i, j) pairs touch is staged once in LDS per
// tile while the next tile's loads are in flight in registers. The products
// are taken transposed, S^T = K Q^T and O^T = V^T P^T: a lane then holds 16
// scores of one query, so the softmax statistics are lane-local up to one
// exchange across the four lane groups, and the probabilities are already
// the B operand of the second product in registers (the 32 keys of a k-step
// are matched to V^T by storing each 32-key block of V^T in that order).
// The K, V^T and band fragments read from LDS serve both query sets.
template <int HD, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_tp_kernel(AttnArgs a) {
  using M_ = MF<bf16_t>;
  constexpr int HDP = HD <= 32 ? 32 : 64;  // head dim padded for MFMA
  constexpr int NQF = HDP / 32;            // k-steps over head dims
  constexpr int NDT = HDP / 16;            // 16-dim tiles of the output
  constexpr int LK = HDP + 8;              // K / band row pitch (bf16)
  constexpr int LV = 64 + 8;               // V^T row pitch
  constexpr int GP = 20;                   // G^T row pitch (fp32), conflict-free both ways
  constexpr bool REL = MODE == ATT_RELPOS;
  // a padded head keeps a row of ones in V^T at dim HD: the O^T product then
  // accumulates each query's softmax denominator with its own rescaling
  constexpr bool ONES = HD < HDP;
  constexpr int QB = 128;                  // query rows per workgroup
  constexpr int NB = REL ? QB + 64 : 0;    // band rows per key tile
  constexpr int CPK = HDP / 8;             // 16-byte chunks per K / band row
  constexpr int NCK = 64 * CPK / 256, NCV = HDP * 8 / 256, NCB = NB * CPK / 256;
  static_assert(MODE != ATT_ROPE, "rotary layers use the latency form");
  __shared__ __align__(16) bf16_t Ks[64 * LK];
  __shared__ __align__(16) bf16_t Vs[HDP * LV];
  __shared__ __align__(16) bf16_t Bs[REL ? NB * LK : 8];
  __shared__ float Gs[REL ? 4 * 80 * GP : 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  // XCD-aware order (bijection over the grid): physical workgroup i runs on
  // XCD i % 8, and XCD x takes a contiguous range of the (stream, head, query
  // block) order, so a stream's K, V^T and Q rows are fetched into one L2
  int iq0, h, b;
  {
    const int gx = gridDim.x, gy = gridDim.y, total = gx * gy * gridDim.z;
    const int pid = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    const int q8 = total / 8, r8 = total % 8, xcd = pid % 8;
    const int t = xcd * q8 + min(xcd, r8) + pid / 8;
    iq0 = (t % gx) * QB;
    h = (t / gx) % gy;
    b = t / (gx * gy);
  }
  const int iw = iq0 + 32 * w;  // this wave's first query row
  const bf16_t* qkv = static_cast<const bf16_t*>(a.qkv);
  const size_t rowbase = (size_t)b * a.W;
  const float sl2 = a.scale * 1.4426950408889634f;
  const bf16_t* vtb = static_cast<const bf16_t*>(a.vt) + (size_t)(b * a.H + h) * HD * a.vpitch;
  const bf16_t* P = static_cast<const bf16_t*>(a.P);

  // ---- Q^T fragments (B operand): column c16 = query iw + 16s + c16, element
  // e of k-step ks = dim 32ks + 8g + e; qb carries the v bias for positions
  bf16x8_t qa[2][NQF], qb[2][NQF];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int qi = iw + 16 * s + c16, qc = min(qi, a.W - 1);
#pragma unroll
    for (int ks = 0; ks < NQF; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      const vec16 raw = *reinterpret_cast<const vec16*>(
          qkv + (rowbase + qc) * a.ldq + a.qoff + h * HD + min(d0, HD - 8));
      const bool live = qi < a.W && d0 < HD;
      float ua[8], va[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wv = raw.w[e / 2];
        const float q = live ? __uint_as_float(e & 1 ? (wv & 0xFFFF0000u) : (wv << 16)) : 0.f;
        ua[e] = q;
        va[e] = q;
        if constexpr (REL) {
          const int dc = min(d0 + e, HD - 1);
          ua[e] += d0 < HD ? a.ub[h * HD + dc] : 0.f;
          va[e] += d0 < HD ? a.vb[h * HD + dc] : 0.f;
        }
      }
      qa[s][ks] = Pack<bf16_t>::make(ua);
      qb[s][ks] = Pack<bf16_t>::make(va);
    }
  }

  // ---- one tile's K, V^T and band chunks into registers (clamped, unconditional)
  vec16 rk[NCK], rv[NCV], rbd[NCB > 0 ? NCB : 1];
  // element offsets in 32 bits (the batch holds at most 64 x 1024 rows of
  // at most 1536 columns, the position table 2047 x 512)
  const bf16_t* kbase = qkv + rowbase * a.ldq + a.koff + h * HD;
  const bf16_t* pbase = P + h * HD;
  auto fetch = [&](int j0) {
#pragma unroll
    for (int i = 0; i < NCK; ++i) {
      const int c = tid + 256 * i, r = c / CPK, q = c % CPK;
      const int j = min(j0 + r, a.W - 1), d = min(8 * q, HD - 8);
      rk[i] = *reinterpret_cast<const vec16*>(kbase + (j * a.ldq + d));
    }
#pragma unroll
    for (int i = 0; i < NCV; ++i) {
      const int c = tid + 256 * i, d = c / 8, q = c % 8;
      rv[i] = *reinterpret_cast<const vec16*>(vtb + (min(d, HD - 1) * a.vpitch +
                                                     min(j0 + 8 * q, a.vpitch - 8)));
    }
#pragma unroll
    for (int i = 0; i < NCB; ++i) {
      const int c = tid + 256 * i, r = c / CPK, q = c % CPK;
      const int pr = min(max(iq0 - j0 - 63 + r + a.p_center, 0), 2 * a.p_center);
      rbd[i] = *reinterpret_cast<const vec16*>(pbase + (pr * a.ldp + 8 * q));
    }
  };
  // zero what lies outside the head, the window or the position table; V^T
  // keys go to their k-slot order (in-block key 16u + 4v + t at 8v + 4u + t)
  // (the masks are workgroup-uniform no-ops except on a tile that crosses
  // the window end or a band that leaves the position table)
  auto stash = [&](int j0) {
#pragma unroll
    for (int i = 0; i < NCK; ++i) {
      const int c = tid + 256 * i, r = c / CPK, q = c % CPK;
      const bool live = 8 * q < HD;
#pragma unroll
      for (int e = 0; e < 4; ++e) rk[i].w[e] = live ? rk[i].w[e] : 0u;
      *reinterpret_cast<vec16*>(&Ks[r * LK + 8 * q]) = rk[i];
    }
    const bool vedge = j0 + 64 > a.W;
#pragma unroll
    for (int i = 0; i < NCV; ++i) {
      const int c = tid + 256 * i, d = c / 8, q = c % 8, j = j0 + 8 * q;
      uint32_t m[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) m[e] = d < HD ? rv[i].w[e] : ONES && d == HD ? 0x3F803F80u : 0u;
      if (vedge) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = j + 2 * e < a.W ? (m[e] & 0xFFFFu) : 0u;
          const uint32_t hi = j + 2 * e + 1 < a.W ? (m[e] & 0xFFFF0000u) : 0u;
          m[e] = lo | hi;
        }
      }
      const int qq = q & 3;
      bf16_t* dst = &Vs[d * LV + 32 * (q >> 2) + 16 * (qq & 1) + 4 * (qq >> 1)];
      *reinterpret_cast<uint2*>(dst) = uint2{m[0], m[1]};
      *reinterpret_cast<uint2*>(dst + 8) = uint2{m[2], m[3]};
    }
    const bool bedge = iq0 - j0 - 63 < -a.p_center || iq0 - j0 - 63 + NB - 1 > a.p_center;
#pragma unroll
    for (int i = 0; i < NCB; ++i) {
      const int c = tid + 256 * i, r = c / CPK, q = c % CPK;
      const int dl = iq0 - j0 - 63 + r;
      if (bedge) {
        const bool live = dl >= -a.p_center && dl <= a.p_center;
#pragma unroll
        for (int e = 0; e < 4; ++e) rbd[i].w[e] = live ? rbd[i].w[e] : 0u;
      }
      *reinterpret_cast<vec16*>(&Bs[r * LK + 8 * q]) = rbd[i];
    }
  };

  // O^T: lane (g, c16) holds dims 16dt + 4g + r of query iw + 16s + c16
  f32x4 O[2][NDT];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[s][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};  // lrow: this lane's keys

  const int n_valid = a.nv ? *a.nv : a.n_valid;
  const int ntile = (n_valid + 63) / 64;
  fetch(0);
  for (int kt = 0; kt < ntile; ++kt) {
    const int j0 = kt * 64;
    __syncthreads();  // every wave is done with the previous tile
    stash(j0);
    __syncthreads();
    // next tile (this one again on the last step: unconditional loads keep the
    // staging arrays in registers), in flight while this tile is used
    fetch(min(j0 + 64, (ntile - 1) * 64));

    // ---- S^T: lane (g, c16) holds keys j0 + 16nt + 4g + r of its query. With
    // relative positions the accumulators start from the position term, so
    // the K Q^T products add onto it.
    f32x4 S[2][4];
    if constexpr (REL) {
      // G^T[rho][c] = p(delta).(q_c + v) with band row 32w + 16s + rho <->
      // delta = (iw + 16s) - j0 - 63 + rho; the score of (query c, key k)
      // takes rho = c - k + 63
      float* G = &Gs[w * 80 * GP];
      bf16x8_t bfr[6][NQF];
#pragma unroll
      for (int bt = 0; bt < 6; ++bt)
#pragma unroll
        for (int ks = 0; ks < NQF; ++ks)
          bfr[bt][ks] = *reinterpret_cast<const bf16x8_t*>(
              &Bs[(32 * w + 16 * bt + c16) * LK + ks * 32 + 8 * g]);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int ct = 0; ct < 5; ++ct) {
          f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NQF; ++ks) acc = M_::mma(bfr[s + ct][ks], qb[s][ks], acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) G[(16 * ct + 4 * g + r) * GP + c16] = acc[r];
        }
        wave_lds_sync();
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            S[s][nt][r] = G[(c16 - 16 * nt - 4 * g - r + 63) * GP + c16];
        wave_lds_sync();  // the next set rewrites G
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        S[0][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        S[1][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int ks = 0; ks < NQF; ++ks) {
        const bf16x8_t kf =
            *reinterpret_cast<const bf16x8_t*>(&Ks[(16 * nt + c16) * LK + ks * 32 + 8 * g]);
        S[0][nt] = M_::mma(kf, qa[0][ks], S[0][nt]);
        S[1][nt] = M_::mma(kf, qa[1][ks], S[1][nt]);
      }

    // ---- online softmax (log2 domain: the running max is kept scaled by
    // scale*log2(e), p = 2^(s*scale*log2(e) - m)); P^T as the B operand of
    // O^T += V^T P^T. Keys past n_valid exist only in the last tile.
    if (j0 + 64 > n_valid) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            S[s][nt][r] = j0 + 16 * nt + 4 * g + r < n_valid ? S[s][nt][r] : -INFINITY;
    }
    bf16x8_t pb[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float mx = -INFINITY;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S[s][nt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrow[s], mx * sl2);
      float rs = 0.f, p[4][4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[nt][r] = __builtin_amdgcn_exp2f(fmaf(S[s][nt][r], sl2, -mnew));
          if constexpr (!ONES) rs += p[nt][r];
        }
      if (__ballot(mnew != mrow[s])) {  // rescale only when some query's max moved
        const float alpha = __builtin_amdgcn_exp2f(mrow[s] - mnew);
        if constexpr (!ONES) lrow[s] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) O[s][dt][r] *= alpha;
      }
      if constexpr (!ONES) lrow[s] += rs;
      mrow[s] = mnew;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = p[2 * ks][e];
          pv[4 + e] = p[2 * ks + 1][e];
        }
        pb[s][ks] = Pack<bf16_t>::make(pv);
      }
    }
    // ---- O^T += V^T P^T (V^T columns past the window or the head are zero)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8_t vf =
            *reinterpret_cast<const bf16x8_t*>(&Vs[(16 * dt + c16) * LV + ks * 32 + 8 * g]);
        O[0][dt] = M_::mma(vf, pb[0][ks], O[0][dt]);
        O[1][dt] = M_::mma(vf, pb[1][ks], O[1][dt]);
      }
  }

  bf16_t* ctx = static_cast<bf16_t*>(a.ctx);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float l;
    if constexpr (ONES) {  // dim HD of query c16 sits in lane group (HD % 16) / 4
      l = __shfl(O[s][HD / 16][HD % 4], 16 * ((HD % 16) / 4) + c16);
    } else {
      l = lrow[s];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
    }
    const int i = iw + 16 * s + c16;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d = 16 * dt + 4 * g;
      if (i < a.W && d < HD) {
        u16x4 u;
#pragma unroll
        for (int r = 0; r < 4; ++r) u[r] = f2bf(O[s][dt][r] / l);
        *reinterpret_cast<u16x4*>(&ctx[(rowbase + i) * a.ldc + h * HD + d]) = u;
      }
    }
  }
}

template <typename T, int NW>
static void launch_attn_nw(const AttnArgs& a, int mode, int hd, hipStream_t s, double fl, double by) {
  dim3 grid((a.W + 15) / 16, a.H, a.B), block(NW * 64);
  if (mode == ATT_RELPOS && hd == 64)
    klaunch(PROF_ATTN, fl, by, attn_kernel<T, 64, ATT_RELPOS, NW>, grid, block, s, a);
  else if (mode == ATT_ROPE && hd == 64)
    klaunch(PROF_ATTN, fl, by, attn_kernel<T, 64, ATT_ROPE, NW>, grid, block, s, a);
  else if (mode == ATT_PLAIN && hd == 24)
    klaunch(PROF_ATTN, fl, by, attn_kernel<T, 24, ATT_PLAIN, NW>, grid, block, s, a);
  else if (mode == ATT_PLAIN && hd == 64)
    klaunch(PROF_ATTN, fl, by, attn_kernel<T, 64, ATT_PLAIN, NW>, grid, block, s, a);
}

// Four waves per workgroup: eight gave no gain for one stream and cost a
// third more time for 64 streams (twice the LDS, fewer workgroups per CU).
// The split of key tiles over waves is fixed, so a stream's result does not
// depend on how many streams share the launch.
template <typename T>
static void launch_attn(const AttnArgs& a, int mode, int hd, hipStream_t s, double fl, double by) {
  launch_attn_nw<T, 4>(a, mode, hd, s, fl, by);
}

// Latency form for single windows and small batches; the throughput form
// once streams x window exceeds 4096 rows (the row count at which the GEMMs
// switch to whole-K loops too).
static bool use_tp(const AttnArgs& a, int mode, int hd, bool bf16) {
  return bf16 && (long long)a.B * a.W > 4096 &&
         ((mode == ATT_RELPOS && hd == 64) || (mode == ATT_PLAIN && hd == 24));
}

void attention(const AttnArgs& a, int mode, int head_dim, bool bf16, hipStream_t s) {
  if (a.W <= 0 || a.B <= 0) return;
  if (a.wo_f && (!bf16 || mode == ATT_PLAIN || head_dim != 64 || a.H * head_dim != 512 ||
                 !a.part || a.M != a.B * a.W || use_tp(a, mode, head_dim, bf16))) {
    flag_launch_failure();  // the fused projection exists only in the latency form
    return;
  }
  // scores (q.k), the relative-position term (q.p(i-j)) and P.V per head,
  // plus the fused output projection (its weights and fp32 partials)
  const double pairs = (double)a.B * a.H * a.W * a.n_valid;
  const double es = bf16 ? 2 : 4;
  const double rows = (double)a.B * a.W;
  const double fl = pairs * 2.0 * head_dim * (mode == ATT_RELPOS ? 3 : 2) +
                    (a.wo_f ? 2.0 * rows * 512 * 512 : 0.0);
  const double by = es * a.B * a.W * a.H * head_dim * 4.0 +
                    (a.wo_f ? 2.0 * 512 * 512 + 4.0 * a.H * rows * 512 : 0.0);
  if (use_tp(a, mode, head_dim, bf16)) {
    dim3 grid((a.W + 127) / 128, a.H, a.B);
    if (mode == ATT_RELPOS)
      klaunch(PROF_ATTN, fl, by, attn_tp_kernel<64, ATT_RELPOS>, grid, dim3(256), s, a);
    else
      klaunch(PROF_ATTN, fl, by, attn_tp_kernel<24, ATT_PLAIN>, grid, dim3(256), s, a);
  } else if (bf16) {
    launch_attn<bf16_t>(a, mode, head_dim, s, fl, by);
  } else {
    launch_attn<float>(a, mode, head_dim, s, fl, by);
  }
}

}  // namespace sf
