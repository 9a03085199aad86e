// Host-side weight generation: canonical tensor lists and the seeded
// random-init (SplitMix64 counter -> two 53-bit uniforms -> Box-Muller).
//
// Tensor i, element e (row-major, PyTorch order):
//   c1 = splitmix64(seed ^ (i<<40) ^ 2e), c2 = splitmix64(seed ^ (i<<40) ^ (2e+1))
//   u1 = ((c1>>11)+1) 2^-53, u2 = (c2>>11) 2^-53, z = sqrt(-2 ln u1) cos(2 pi u2)
// kind 'w': 0.02 z; 'b': 0 (full-random: 0.02 z); 'g': 1 (full-random: 1+0.02 z).
// SplitMix64 is Steele, Lea and Flood's generator with Vigna's constants.
#include "host.h"

#include <cmath>
#include <thread>

namespace sfh {

static void add(std::vector<TSpec>& t, const std::string& n, std::vector<int64_t> shape, char k) {
  t.push_back(TSpec{n, std::move(shape), k});
}

std::vector<TSpec> sortformer_list(int S) {
  std::vector<TSpec> t;
  add(t, "pre.conv0.w", {256, 1, 3, 3}, 'w');
  add(t, "pre.conv0.b", {256}, 'b');
  for (int k = 1; k <= 2; ++k) {
    std::string p = "pre.dw" + std::to_string(k);
    add(t, p + ".w", {256, 1, 3, 3}, 'w');
    add(t, p + ".b", {256}, 'b');
    p = "pre.pw" + std::to_string(k);
    add(t, p + ".w", {256, 256, 1, 1}, 'w');
    add(t, p + ".b", {256}, 'b');
  }
  add(t, "pre.out.w", {512, 4096}, 'w');
  add(t, "pre.out.b", {512}, 'b');
  for (int l = 0; l < 17; ++l) {
    const std::string p = "conf" + std::to_string(l) + ".";
    auto ff = [&](const std::string& f) {
      add(t, p + f + ".ln.g", {512}, 'g');
      add(t, p + f + ".ln.b", {512}, 'b');
      add(t, p + f + ".w1", {2048, 512}, 'w');
      add(t, p + f + ".b1", {2048}, 'b');
      add(t, p + f + ".w2", {512, 2048}, 'w');
      add(t, p + f + ".b2", {512}, 'b');
    };
    ff("ff1");
    add(t, p + "att.ln.g", {512}, 'g');
    add(t, p + "att.ln.b", {512}, 'b');
    for (const char* m : {"q", "k", "v", "o"}) {
      add(t, p + "att.w" + m, {512, 512}, 'w');
      add(t, p + "att.b" + m, {512}, 'b');
    }
    add(t, p + "att.wpos", {512, 512}, 'w');
    add(t, p + "att.u", {8, 64}, 'w');
    add(t, p + "att.v", {8, 64}, 'w');
    add(t, p + "conv.ln.g", {512}, 'g');
    add(t, p + "conv.ln.b", {512}, 'b');
    add(t, p + "conv.pw1.w", {1024, 512}, 'w');
    add(t, p + "conv.pw1.b", {1024}, 'b');
    add(t, p + "conv.dw.w", {512, 9}, 'w');
    add(t, p + "conv.dw.b", {512}, 'b');
    add(t, p + "conv.bn.g", {512}, 'g');
    add(t, p + "conv.bn.b", {512}, 'b');
    add(t, p + "conv.bn.mean", {512}, 'b');
    add(t, p + "conv.bn.var", {512}, 'g');
    add(t, p + "conv.pw2.w", {512, 512}, 'w');
    add(t, p + "conv.pw2.b", {512}, 'b');
    ff("ff2");
    add(t, p + "out_ln.g", {512}, 'g');
    add(t, p + "out_ln.b", {512}, 'b');
  }
  add(t, "proj.w", {192, 512}, 'w');
  add(t, "proj.b", {192}, 'b');
  for (int l = 0; l < 18; ++l) {
    const std::string p = "tf" + std::to_string(l) + ".";
    for (const char* m : {"q", "k", "v", "o"}) {
      add(t, p + "w" + m, {192, 192}, 'w');
      add(t, p + "b" + m, {192}, 'b');
    }
    add(t, p + "ln1.g", {192}, 'g');
    add(t, p + "ln1.b", {192}, 'b');
    add(t, p + "w1", {768, 192}, 'w');
    add(t, p + "b1", {768}, 'b');
    add(t, p + "w2", {192, 768}, 'w');
    add(t, p + "b2", {192}, 'b');
    add(t, p + "ln2.g", {192}, 'g');
    add(t, p + "ln2.b", {192}, 'b');
  }
  add(t, "head.w1", {192, 192}, 'w');
  add(t, "head.b1", {192}, 'b');
  add(t, "head.w2", {S, 192}, 'w');
  add(t, "head.b2", {S}, 'b');
  return t;
}

std::vector<TSpec> nemotron_list(int S) {
  std::vector<TSpec> t;
  add(t, "in.w", {512, 1024}, 'w');
  add(t, "in.b", {512}, 'b');
  for (int l = 0; l < 31; ++l) {
    const std::string p = "rl" + std::to_string(l) + ".";
    add(t, p + "ln1.g", {512}, 'g');
    add(t, p + "ln1.b", {512}, 'b');
    for (const char* m : {"q", "k", "v", "o"}) {
      add(t, p + "w" + m, {512, 512}, 'w');
      add(t, p + "b" + m, {512}, 'b');
    }
    add(t, p + "ln2.g", {512}, 'g');
    add(t, p + "ln2.b", {512}, 'b');
    add(t, p + "w1", {2048, 512}, 'w');
    add(t, p + "b1", {2048}, 'b');
    add(t, p + "w2", {512, 2048}, 'w');
    add(t, p + "b2", {512}, 'b');
  }
  add(t, "final_ln.g", {512}, 'g');
  add(t, "final_ln.b", {512}, 'b');
  add(t, "head.w", {S, 512}, 'w');
  add(t, "head.b", {S}, 'b');
  add(t, "up.w", {S, S, 8}, 'w');
  add(t, "up.b", {S}, 'b');
  return t;
}

static inline uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static void gen_range(uint64_t seed, int index, char kind, bool full, int64_t e0, int64_t e1,
                      float* out) {
  const uint64_t base = seed ^ ((uint64_t)index << 40);
  for (int64_t e = e0; e < e1; ++e) {
    if (kind != 'w' && !full) {
      out[e] = kind == 'g' ? 1.0f : 0.0f;
      continue;
    }
    const uint64_t c1 = splitmix64(base ^ (uint64_t)(2 * e));
    const uint64_t c2 = splitmix64(base ^ (uint64_t)(2 * e + 1));
    const double u1 = ((double)(c1 >> 11) + 1.0) * 0x1p-53;
    const double u2 = (double)(c2 >> 11) * 0x1p-53;
    const double z = std::sqrt(-2.0 * std::log(u1)) * std::cos(2.0 * M_PI * u2);
    out[e] = kind == 'g' ? (float)(1.0 + 0.02 * z) : (float)(0.02 * z);
  }
}

void generate(const std::vector<TSpec>& list, uint64_t seed, bool full,
              std::vector<std::vector<float>>& out) {
  out.resize(list.size());
  for (size_t i = 0; i < list.size(); ++i) out[i].assign(list[i].numel(), 0.f);
  unsigned nt = std::thread::hardware_concurrency();
  if (nt == 0) nt = 4;
  if (nt > 16) nt = 16;
  // split the concatenation of all tensors into equal element ranges
  int64_t total = 0;
  for (auto& t : list) total += t.numel();
  std::vector<std::thread> th;
  for (unsigned w = 0; w < nt; ++w) {
    th.emplace_back([&, w]() {
      const int64_t lo = total * w / nt, hi = total * (w + 1) / nt;
      int64_t off = 0;
      for (size_t i = 0; i < list.size(); ++i) {
        const int64_t n = list[i].numel();
        const int64_t a = std::max(lo, off), b = std::min(hi, off + n);
        if (a < b) gen_range(seed, (int)i, list[i].kind, full, a - off, b - off, out[i].data());
        off += n;
      }
    });
  }
  for (auto& t : th) t.join();
}

}  // namespace sfh
