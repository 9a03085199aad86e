"""Seeded random-init weights (the models are run with random weights; no
trained checkpoint is used).

Generator: tensor number ``i`` of the canonical list, element ``e`` of its
row-major (PyTorch-order) flattening:

    c1 = splitmix64(seed ^ (i << 40) ^ (2e)),  c2 = splitmix64(seed ^ (i << 40) ^ (2e+1))
    u1 = ((c1 >> 11) + 1) * 2^-53   in (0, 1]
    u2 =  (c2 >> 11)      * 2^-53   in [0, 1)
    z  = sqrt(-2 ln u1) * cos(2 pi u2)          (Box-Muller, in float64)

splitmix64 is the output mix of Steele, Lea and Flood's SplitMix generator
(Vigna's 64-bit constants): add the golden gamma 0x9E3779B97F4A7C15, then two
xor-shift-multiply rounds (30, 0xBF58476D1CE4E5B9; 27, 0x94D049BB133111EB)
and a final xor-shift by 31.

Init rule per tensor kind ("Weights ~N(0, 0.02) ... LayerNorm gamma=1,
beta=0" in the workload description; biases zero is the stated reading):
  "w" (matrices, conv kernels, pos-bias u/v):   fp32(0.02 z)
  "b" (biases, LN/BN beta, BN running mean):    0          | full-random: fp32(0.02 z)
  "g" (LN/BN gamma, BN running var):            1          | full-random: fp32(1 + 0.02 z)

The canonical tensor lists below follow the architecture of the "Streaming
Sortformer Diarizer" model card (Pipeline, Model Parameters) and of the
Nemotron-3-Diarization model-card summary in the ExecuTorch issue.
"""
from __future__ import annotations

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(x: np.ndarray) -> np.ndarray:
    z = x.astype(np.uint64) + _GAMMA
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def normal_draws(seed: int, tensor_index: int, count: int) -> np.ndarray:
    """float64 standard normals for elements 0..count-1 of one tensor."""
    base = np.uint64(seed) ^ (np.uint64(tensor_index) << np.uint64(40))
    e2 = np.arange(count, dtype=np.uint64) * np.uint64(2)
    c1 = splitmix64(base ^ e2)
    c2 = splitmix64(base ^ (e2 + np.uint64(1)))
    u1 = ((c1 >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = (c2 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def sortformer_tensors(n_spk: int = 4):
    """Canonical (name, shape, kind) list of the 4-speaker Sortformer.

    Pipeline: dw-striding ConvSubsampling (conv0 1->256 3x3/2, then twice
    depthwise 3x3/2 + pointwise 256->256), Linear 4096->512; 17 conformer
    layers (macaron FFN 512->2048, rel-pos MHSA 8x64 with u/v biases and a
    bias-free positional projection, conv module pw 512->1024, GLU,
    depthwise k=9, BatchNorm, pw 512->512, output LN); Linear 512->192;
    18 post-LN transformer layers (8 heads, FFN 768); head 192->192->n_spk.
    """
    t = []
    t += [("pre.conv0.w", (256, 1, 3, 3), "w"), ("pre.conv0.b", (256,), "b")]
    for k in (1, 2):
        t += [(f"pre.dw{k}.w", (256, 1, 3, 3), "w"), (f"pre.dw{k}.b", (256,), "b"),
              (f"pre.pw{k}.w", (256, 256, 1, 1), "w"), (f"pre.pw{k}.b", (256,), "b")]
    t += [("pre.out.w", (512, 4096), "w"), ("pre.out.b", (512,), "b")]
    for l in range(17):
        p = f"conf{l}."
        t += [(p + "ff1.ln.g", (512,), "g"), (p + "ff1.ln.b", (512,), "b"),
              (p + "ff1.w1", (2048, 512), "w"), (p + "ff1.b1", (2048,), "b"),
              (p + "ff1.w2", (512, 2048), "w"), (p + "ff1.b2", (512,), "b")]
        t += [(p + "att.ln.g", (512,), "g"), (p + "att.ln.b", (512,), "b")]
        for m in ("q", "k", "v", "o"):
            t += [(p + f"att.w{m}", (512, 512), "w"), (p + f"att.b{m}", (512,), "b")]
        t += [(p + "att.wpos", (512, 512), "w"),
              (p + "att.u", (8, 64), "w"), (p + "att.v", (8, 64), "w")]
        t += [(p + "conv.ln.g", (512,), "g"), (p + "conv.ln.b", (512,), "b"),
              (p + "conv.pw1.w", (1024, 512), "w"), (p + "conv.pw1.b", (1024,), "b"),
              (p + "conv.dw.w", (512, 9), "w"), (p + "conv.dw.b", (512,), "b"),
              (p + "conv.bn.g", (512,), "g"), (p + "conv.bn.b", (512,), "b"),
              (p + "conv.bn.mean", (512,), "b"), (p + "conv.bn.var", (512,), "g"),
              (p + "conv.pw2.w", (512, 512), "w"), (p + "conv.pw2.b", (512,), "b")]
        t += [(p + "ff2.ln.g", (512,), "g"), (p + "ff2.ln.b", (512,), "b"),
              (p + "ff2.w1", (2048, 512), "w"), (p + "ff2.b1", (2048,), "b"),
              (p + "ff2.w2", (512, 2048), "w"), (p + "ff2.b2", (512,), "b")]
        t += [(p + "out_ln.g", (512,), "g"), (p + "out_ln.b", (512,), "b")]
    t += [("proj.w", (192, 512), "w"), ("proj.b", (192,), "b")]
    for l in range(18):
        p = f"tf{l}."
        for m in ("q", "k", "v", "o"):
            t += [(p + f"w{m}", (192, 192), "w"), (p + f"b{m}", (192,), "b")]
        t += [(p + "ln1.g", (192,), "g"), (p + "ln1.b", (192,), "b"),
              (p + "w1", (768, 192), "w"), (p + "b1", (768,), "b"),
              (p + "w2", (192, 768), "w"), (p + "b2", (192,), "b"),
              (p + "ln2.g", (192,), "g"), (p + "ln2.b", (192,), "b")]
    t += [("head.w1", (192, 192), "w"), ("head.b1", (192,), "b"),
          ("head.w2", (n_spk, 192), "w"), ("head.b2", (n_spk,), "b")]
    return t


def nemotron_tensors(n_spk: int = 8):
    """Canonical list of the Nemotron-3-style variant: Linear 1024->512 on
    8x-stacked mel, 31 pre-LN RoPE layers (8x64 heads, GELU FFN 2048),
    final LN, head Linear 512->n_spk, ConvTranspose1d(n_spk, n_spk, k=8, s=8)."""
    t = [("in.w", (512, 1024), "w"), ("in.b", (512,), "b")]
    for l in range(31):
        p = f"rl{l}."
        t += [(p + "ln1.g", (512,), "g"), (p + "ln1.b", (512,), "b")]
        for m in ("q", "k", "v", "o"):
            t += [(p + f"w{m}", (512, 512), "w"), (p + f"b{m}", (512,), "b")]
        t += [(p + "ln2.g", (512,), "g"), (p + "ln2.b", (512,), "b"),
              (p + "w1", (2048, 512), "w"), (p + "b1", (2048,), "b"),
              (p + "w2", (512, 2048), "w"), (p + "b2", (512,), "b")]
    t += [("final_ln.g", (512,), "g"), ("final_ln.b", (512,), "b"),
          ("head.w", (n_spk, 512), "w"), ("head.b", (n_spk,), "b"),
          ("up.w", (n_spk, n_spk, 8), "w"), ("up.b", (n_spk,), "b")]
    return t


# Matrices that the bf16 path feeds to bf16 GEMMs; these (and only these)
# are rounded to bf16 when the oracle models a bf16 configuration. The
# direct convolutions (conv0, depthwise), the pos-bias vectors and the small
# speaker heads stay fp32.
_SF_GEMM_LEAVES = {"ff1.w1", "ff1.w2", "ff2.w1", "ff2.w2", "att.wq", "att.wk",
                   "att.wv", "att.wo", "att.wpos", "conv.pw1.w", "conv.pw2.w"}


def is_gemm_matrix(name: str, arch: str) -> bool:
    if arch == "sortformer":
        if name in ("pre.pw1.w", "pre.pw2.w", "pre.out.w", "proj.w"):
            return True
        if name.startswith("conf"):
            return name.split(".", 1)[1] in _SF_GEMM_LEAVES
        if name.startswith("tf"):
            return name.split(".", 1)[1] in ("wq", "wk", "wv", "wo", "w1", "w2")
        return False
    if name == "in.w":
        return True
    if name.startswith("rl"):
        return name.split(".", 1)[1] in ("wq", "wk", "wv", "wo", "w1", "w2")
    return False


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), as float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    r = ((bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32).reshape(f.shape)


def make_weights(arch: str = "sortformer", seed: int = 0, full_random: bool = False,
                 bf16: bool = False, n_spk: int | None = None) -> dict:
    """Dict name -> float64 array (fp32 values; bf16 values for GEMM matrices
    when ``bf16``)."""
    if arch == "sortformer":
        tl = sortformer_tensors(4 if n_spk is None else n_spk)
    elif arch == "nemotron":
        tl = nemotron_tensors(8 if n_spk is None else n_spk)
    else:
        raise ValueError(arch)
    out = {}
    for i, (name, shape, kind) in enumerate(tl):
        n = int(np.prod(shape))
        if kind == "w" or full_random:
            z = normal_draws(seed, i, n)
        if kind == "w":
            v = (0.02 * z).astype(np.float32)
        elif kind == "b":
            v = (0.02 * z).astype(np.float32) if full_random else np.zeros(n, np.float32)
        elif kind == "g":
            v = (1.0 + 0.02 * z).astype(np.float32) if full_random else np.ones(n, np.float32)
        else:
            raise ValueError(kind)
        v = v.reshape(shape)
        if bf16 and is_gemm_matrix(name, arch):
            v = bf16_round(v)
        out[name] = v.astype(np.float64)
    return out


def param_count(arch: str = "sortformer") -> int:
    """Trainable parameters (BatchNorm running statistics excluded)."""
    tl = sortformer_tensors() if arch == "sortformer" else nemotron_tensors()
    return sum(int(np.prod(s)) for n, s, k in tl
               if not (n.endswith("bn.mean") or n.endswith("bn.var")))
