// Multi-head self-attention over one encoder window, flash-style.
//
// One single-wave workgroup = (16 query rows, head, stream), so a window of
// a few hundred frames still spreads over a few hundred workgroups. Key/value
// tiles of 64 frames are staged through LDS (V comes already transposed per
// head from the QKV projection, so both MFMA operands are K-contiguous and
// staging is plain 16-byte copies); the next tile's K, V (and position band)
// are fetched into registers while the current tile is computed. Scores, the
// online softmax (running max/sum in fp32, exp2 domain) and the P.V product
// stay on the matrix cores and in registers.
//
// Modes:
//  ATT_RELPOS  FastConformer relative-position attention ("Streaming
//    Sortformer Diarizer" card, torch.export Fixes 6: rel_shift). The score of
//    query i and key j is [(q_i+u).k_j + (q_i+v).p(i-j)]/sqrt(d). The
//    projections p(delta) are input-independent and precomputed for every
//    delta; per key tile the 80-row band of p that the tile's (i, j) pairs
//    touch is staged in LDS, one more MFMA product G = (q+v).band^T is formed,
//    and the shift is done by indexing G at column i-j+63 — no padded score
//    matrix is materialised.
//  ATT_ROPE    rotary embedding on q and k (rotate-half, positions = window
//    index, which restart at every chunk) for the Nemotron-style layers.
//  ATT_PLAIN   standard scaled dot-product attention (transformer, d=24,
//    zero-padded to 32 for the MFMA K dimension).
// Keys at index >= n_valid are right padding and are masked.
#include "kernels.h"

namespace sf {

// A workgroup here is one wave: LDS writes by some lanes become visible to
// the others once the wave's LDS operations have completed, so a wait on
// the LDS counter replaces a workgroup barrier (whose fence would also drain
// the prefetched global loads).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt/expcnt unconstrained
  __builtin_amdgcn_wave_barrier();
}

template <typename T> struct Pack;
template <> struct Pack<float> {
  __device__ static float make(const float* v) { return v[0]; }
};
template <> struct Pack<bf16_t> {
  __device__ static bf16x8_t make(const float* v) {
    u16x8 u;
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = f2bf(v[e]);
    return __builtin_bit_cast(bf16x8_t, u);
  }
};

template <typename T, int HD, int MODE>
__global__ __launch_bounds__(64) void attn_kernel(AttnArgs a) {
  using M_ = MF<T>;
  constexpr int KI = M_::KI;
  constexpr int EPF = KI / 4;              // elements per fragment per lane
  constexpr int HDP = HD <= 32 ? 32 : 64;  // padded head dim
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int LDK = HDP + VEC;
  constexpr int LDV = 64 + VEC;
  constexpr int NQF = HDP / KI;
  constexpr int CPR = HDP / VEC;           // 16-byte chunks per staged row
  constexpr bool REL = MODE == ATT_RELPOS;
  constexpr bool ROPE = MODE == ATT_ROPE;
  static_assert(!ROPE || HD == 64, "rotary layers use 64-dim heads");
  constexpr int NB = 80;                   // band rows: 16 queries + 64 keys - 1, padded
  constexpr int KCH = ROPE ? 64 * (CPR / 2) / 64 : 64 * CPR / 64;  // K chunks (pairs) per lane
  constexpr int VCPR = 64 / VEC;           // chunks per V^T row (64 keys)
  constexpr int VCH = HDP * VCPR / 64;
  constexpr int BCH = REL ? NB * CPR / 64 : 1;
  __shared__ __align__(16) T Ks[64 * LDK];
  __shared__ __align__(16) T Vt[HDP * LDV];
  __shared__ __align__(16) T Pb[REL ? NB * LDK : VEC];
  __shared__ float Gs[REL ? 16 * 81 : 1];
  __shared__ __align__(16) T Ps[16 * LDV];

  const int lane = threadIdx.x, g = lane >> 4, c16 = lane & 15;
  const int iq0 = blockIdx.x * 16, h = blockIdx.y, b = blockIdx.z;
  const T* qkv = static_cast<const T*>(a.qkv);
  const size_t rowbase = (size_t)b * a.W;
  const float sl2 = a.scale * 1.4426950408889634f;

  // ---- query fragments for row iq0+c16: element e of fragment ks is dim
  // ks*KI + EPF*g + e.
  typename M_::frag qa[NQF], qb[NQF];
  {
    const int qi = iq0 + c16;
    const int qc = min(qi, a.W - 1);
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
      const int pos = qi < a.W ? qi : 0;
#pragma unroll
      for (int ks = 0; ks < HALF; ++ks)
#pragma unroll
        for (int e = 0; e < EPF; ++e) {
          const int d = ks * KI + EPF * g + e;
          const float c = a.rope[(pos * 32 + d) * 2], s = a.rope[(pos * 32 + d) * 2 + 1];
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

  // ---- register staging of one key tile (K, V and the position band); the
  // next tile is fetched while the current one is being computed.
  const vec16 zero{{0u, 0u, 0u, 0u}};
  vec16 kr[KCH], kr2[ROPE ? KCH : 1], vr[VCH], br[BCH];
  // Loads are unconditional (clamped rows/chunks) so they all issue back to
  // back; out-of-range chunks are zeroed by the selects in `mask`.
  auto fetch = [&](int j0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int idx = lane + 64 * i;
      const int r = ROPE ? idx / (CPR / 2) : idx / CPR, c = ROPE ? idx % (CPR / 2) : idx % CPR;
      const int j = min(j0 + r, a.W - 1), d0 = min(c * VEC, HD - VEC);
      const size_t base = (rowbase + j) * a.ldq + a.koff + h * HD + d0;
      kr[i] = *reinterpret_cast<const vec16*>(qkv + base);
      if constexpr (ROPE) kr2[i] = *reinterpret_cast<const vec16*>(qkv + base + 32);
    }
    const T* vt = static_cast<const T*>(a.vt) + (size_t)(b * a.H + h) * HD * a.vpitch;
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int idx = lane + 64 * i, d = min(idx / VCPR, HD - 1);
      const int k0 = min(j0 + (idx % VCPR) * VEC, a.vpitch - VEC);
      vr[i] = *reinterpret_cast<const vec16*>(vt + (size_t)d * a.vpitch + k0);
    }
    if constexpr (REL) {
      const int dbase = iq0 - j0 - 63 + a.p_center;
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        const int idx = lane + 64 * i, r = idx / CPR, d0 = min((idx % CPR) * VEC, HD - VEC);
        const int trow = min(max(dbase + r, 0), 2 * a.p_center);
        br[i] = *reinterpret_cast<const vec16*>(static_cast<const T*>(a.P) + (size_t)trow * a.ldp +
                                                h * HD + d0);
      }
    }
  };
  auto zap = [](vec16& v, bool live) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v.w[q] = live ? v.w[q] : 0u;
  };
  auto mask = [&](int j0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int idx = lane + 64 * i;
      const int r = ROPE ? idx / (CPR / 2) : idx / CPR, c = ROPE ? idx % (CPR / 2) : idx % CPR;
      zap(kr[i], j0 + r < a.W && c * VEC < HD);
      if constexpr (ROPE) zap(kr2[i], j0 + r < a.W);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {  // dims past HD and keys past W are zero
      const int idx = lane + 64 * i, k0 = j0 + (idx % VCPR) * VEC;
      T* ve = reinterpret_cast<T*>(&vr[i]);
      const bool dl = idx / VCPR < HD && k0 + VEC <= a.vpitch;
#pragma unroll
      for (int e = 0; e < VEC; ++e) ve[e] = (dl && k0 + e < a.W) ? ve[e] : from_f<T>(0.f);
    }
    if constexpr (REL) {
      const int dbase = iq0 - j0 - 63 + a.p_center;
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        const int idx = lane + 64 * i, trow = dbase + idx / CPR;
        zap(br[i], trow >= 0 && trow <= 2 * a.p_center && (idx % CPR) * VEC < HD);
      }
    }
  };
  auto stash = [&](int j0) {
    mask(j0);
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int idx = lane + 64 * i;
      const int r = ROPE ? idx / (CPR / 2) : idx / CPR, c = ROPE ? idx % (CPR / 2) : idx % CPR;
      const int d0 = c * VEC;
      if constexpr (ROPE) {
        const T* k1e = reinterpret_cast<const T*>(&kr[i]);
        const T* k2e = reinterpret_cast<const T*>(&kr2[i]);
        const int pos = j0 + r < a.W ? j0 + r : 0;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float c_ = a.rope[(pos * 32 + d0 + e) * 2], s_ = a.rope[(pos * 32 + d0 + e) * 2 + 1];
          const float x1 = to_f<T>(k1e[e]), x2 = to_f<T>(k2e[e]);
          Ks[r * LDK + d0 + e] = from_f<T>(x1 * c_ - x2 * s_);
          Ks[r * LDK + d0 + 32 + e] = from_f<T>(x2 * c_ + x1 * s_);
        }
      } else {
        *reinterpret_cast<vec16*>(&Ks[r * LDK + d0]) = kr[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int idx = lane + 64 * i;
      *reinterpret_cast<vec16*>(&Vt[(idx / VCPR) * LDV + (idx % VCPR) * VEC]) = vr[i];
    }
    if constexpr (REL) {
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        const int idx = lane + 64 * i, r = idx / CPR, d0 = (idx % CPR) * VEC;
        *reinterpret_cast<vec16*>(&Pb[r * LDK + d0]) = br[i];
      }
    }
  };

  f32x4 O[HDP / 16];
#pragma unroll
  for (int dt = 0; dt < HDP / 16; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { mrow[r] = -INFINITY; lrow[r] = 0.f; }

  const int ntile = (a.n_valid + 63) / 64;
  fetch(0);
  for (int kt = 0; kt < ntile; ++kt) {
    const int j0 = kt * 64;
    wave_lds_sync();
    stash(j0);
    wave_lds_sync();
    if (kt + 1 < ntile) fetch(j0 + 64);

    // ---- scores
    f32x4 S[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      S[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NQF; ++ks)
        S[nt] = M_::mma(qa[ks], M_::ld(&Ks[(16 * nt + c16) * LDK + ks * KI], lane), S[nt]);
    }
    if constexpr (REL) {
      // G[i][c] = (q_i+v).band[c], band row c <-> relative distance
      // iq0-j0-63+c; the score of (i, j) takes column i-j+63.
#pragma unroll
      for (int ct = 0; ct < 5; ++ct) {
        f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NQF; ++ks)
          acc = M_::mma(qb[ks], M_::ld(&Pb[(16 * ct + c16) * LDK + ks * KI], lane), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) Gs[(4 * g + r) * 81 + 16 * ct + c16] = acc[r];
      }
      wave_lds_sync();
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[nt][r] += Gs[(4 * g + r) * 81 + (4 * g + r) - (16 * nt + c16) + 63];
    }

    // ---- online softmax (log2 domain)
    float mx[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) mx[r] = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const bool valid = j0 + 16 * nt + c16 < a.n_valid;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        S[nt][r] = valid ? S[nt][r] * sl2 : -INFINITY;
        mx[r] = fmaxf(mx[r], S[nt][r]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mnew = fmaxf(mrow[r], group16_max(mx[r]));
      const float alpha = exp2f(mrow[r] - mnew);
      float rs = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float p = exp2f(S[nt][r] - mnew);
        rs += p;
        Ps[(4 * g + r) * LDV + 16 * nt + c16] = from_f<T>(p);
      }
      lrow[r] = lrow[r] * alpha + group16_sum(rs);
      mrow[r] = mnew;
#pragma unroll
      for (int dt = 0; dt < HDP / 16; ++dt) O[dt][r] *= alpha;
    }
    wave_lds_sync();
    // ---- O += P.V
#pragma unroll
    for (int dt = 0; dt < HDP / 16; ++dt)
#pragma unroll
      for (int ks = 0; ks < 64 / KI; ++ks)
        O[dt] = M_::mma(M_::ld(&Ps[c16 * LDV + ks * KI], lane),
                        M_::ld(&Vt[(16 * dt + c16) * LDV + ks * KI], lane), O[dt]);
  }

  T* ctx = static_cast<T*>(a.ctx);
#pragma unroll
  for (int dt = 0; dt < HDP / 16; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = iq0 + 4 * g + r, d = 16 * dt + c16;
      if (i < a.W && d < HD) ctx[(rowbase + i) * a.ldc + h * HD + d] = from_f<T>(O[dt][r] / lrow[r]);
    }
}

template <typename T>
static void launch_attn(const AttnArgs& a, int mode, int hd, hipStream_t s) {
  dim3 grid((a.W + 15) / 16, a.H, a.B);
  if (mode == ATT_RELPOS && hd == 64)
    hipLaunchKernelGGL((attn_kernel<T, 64, ATT_RELPOS>), grid, dim3(64), 0, s, a);
  else if (mode == ATT_ROPE && hd == 64)
    hipLaunchKernelGGL((attn_kernel<T, 64, ATT_ROPE>), grid, dim3(64), 0, s, a);
  else if (mode == ATT_PLAIN && hd == 24)
    hipLaunchKernelGGL((attn_kernel<T, 24, ATT_PLAIN>), grid, dim3(64), 0, s, a);
  else if (mode == ATT_PLAIN && hd == 64)
    hipLaunchKernelGGL((attn_kernel<T, 64, ATT_PLAIN>), grid, dim3(64), 0, s, a);
}

void attention(const AttnArgs& a, int mode, int head_dim, bool bf16, hipStream_t s) {
  if (a.W <= 0 || a.B <= 0) return;
  // scores (q.k), the relative-position term (q.p(i-j)) and P.V per head
  const double pairs = (double)a.B * a.H * a.W * a.n_valid;
  const double es = bf16 ? 2 : 4;
  ProfScope ps(PROF_ATTN, s, pairs * 2.0 * head_dim * (mode == ATT_RELPOS ? 3 : 2),
               es * a.B * a.W * a.H * head_dim * 4.0);
  if (bf16) launch_attn<bf16_t>(a, mode, head_dim, s);
  else launch_attn<float>(a, mode, head_dim, s);
}

}  // namespace sf
