"""Seeded synthetic inputs for the Lightweight DC layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the HIP path (tests, bench) and the CPU oracle consume
the arrays it returns, so the two sides always see bit-identical inputs.

Shapes follow the GPT-2 small attention block the layer sits in: 6 heads of
head_dim 128 (model_dim 768), from gsyq.cn news 358785, section 7.1 "QK bank".
The 112-token window is the one the AITNT page ("一个国产AI小透明，连续两次刷新
NanoGPT Speedrun世界纪录", section "第二刀-砍层内", Lightweight DC paragraph)
gives.  The pages train on FineWeb; no dataset is available or needed, so the
token stream is a synthetic concatenation of documents whose length mix is
stated per workload below.

Draw order for every workload (one numpy PCG64 stream per seed):
document lengths, Q, K, V, C, G, dO.  Values are drawn in float32 and, for
bf16 workloads, rounded to bf16 with round-to-nearest-even; the rounded values
(held exactly in float32 arrays) are what both sides receive.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

WINDOW = 112


# ----------------------------------------------------------------------------
# bf16 storage helpers (round-to-nearest-even on the float32 bit pattern)
# ----------------------------------------------------------------------------
def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (RNE) and return the 16-bit patterns."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value, returned as float32."""
    return bf16_bits_to_f32(bf16_bits(x32))


# ----------------------------------------------------------------------------
# document streams
# ----------------------------------------------------------------------------
def _lengths_until(rng: np.random.Generator, T: int, draw) -> np.ndarray:
    chunks = []
    total = 0
    while total < T:
        n = max(16, T // 64)
        ls = draw(rng, n)
        chunks.append(ls)
        total += int(ls.sum())
    ls = np.concatenate(chunks)
    cs = np.cumsum(ls)
    ndoc = int(np.searchsorted(cs, T)) + 1  # first prefix reaching T
    ls = ls[:ndoc].copy()
    ls[-1] -= int(cs[ndoc - 1]) - T  # truncate the last document
    return ls


def doc_ids_from_lengths(lengths: np.ndarray) -> np.ndarray:
    return np.repeat(np.arange(len(lengths), dtype=np.int32), lengths).astype(np.int32)


def geometric_docs(rng, T: int, mean: float) -> np.ndarray:
    """Lengths ~ Geometric(p = 1/mean) on {1, 2, ...}; a new document starts at
    each drawn end-of-sequence token."""
    return doc_ids_from_lengths(
        _lengths_until(rng, T, lambda r, n: r.geometric(1.0 / mean, size=n).astype(np.int64)))


def uniform_docs(rng, T: int, lo: int, hi: int) -> np.ndarray:
    """Lengths ~ U{lo..hi} (inclusive)."""
    return doc_ids_from_lengths(
        _lengths_until(rng, T, lambda r, n: r.integers(lo, hi + 1, size=n).astype(np.int64)))


# ----------------------------------------------------------------------------
# workload container
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    T: int
    H: int
    d: int
    window: int
    dtype: str          # "bf16" or "f32": storage type of q, k, v, do and o
    scale: float
    q: np.ndarray       # [T, H, d] float32 (values representable in `dtype`)
    k: np.ndarray
    v: np.ndarray
    c: np.ndarray       # [T, H] float32
    g: np.ndarray       # [T, H] float32
    doc: np.ndarray     # [T] int32
    do: Optional[np.ndarray] = None  # [T, H, d] float32 (representable in `dtype`)
    recipe: str = ""

    def slice(self, lo: int, hi: int) -> "Workload":
        """Tokens [lo, hi) as a workload of its own (views, no copies)."""
        return dataclasses.replace(
            self, name=f"{self.name}[{lo}:{hi}]", T=hi - lo,
            q=self.q[lo:hi], k=self.k[lo:hi], v=self.v[lo:hi],
            c=self.c[lo:hi], g=self.g[lo:hi], doc=self.doc[lo:hi],
            do=None if self.do is None else self.do[lo:hi])

    def torch_inputs(self, device="cuda", with_do=True):
        """The workload as torch tensors on `device` (q, k, v, do in the
        storage dtype; c, g float32; doc int32)."""
        import torch
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32

        def big(x):
            if self.dtype == "bf16":
                bits = bf16_bits(x)
                return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
            return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)

        out = dict(q=big(self.q), k=big(self.k), v=big(self.v),
                   c=torch.from_numpy(np.ascontiguousarray(self.c)).to(device),
                   g=torch.from_numpy(np.ascontiguousarray(self.g)).to(device),
                   doc=torch.from_numpy(np.ascontiguousarray(self.doc)).to(device))
        if with_do and self.do is not None:
            out["do"] = big(self.do)
        assert out["q"].dtype == tdt
        return out


def _normal(rng, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _rms_rows(x: np.ndarray) -> np.ndarray:
    """Each (t, h) row divided by its root mean square: the rows a QK-norm
    producer hands over."""
    ms = np.mean(np.square(x, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
    return (x / np.sqrt(ms)).astype(np.float32)


def make_workload(T: int, H: int, d: int, *, window: int = WINDOW, dtype: str = "bf16",
                  seed: int = 0, docs=("geometric", 1024), qk_rms: bool = True,
                  c_kind: str = "normal0.5", g_kind: str = "u0.5-1.5", with_do: bool = True,
                  scale: Optional[float] = None, name: Optional[str] = None) -> Workload:
    """Generic seeded workload.

    docs:   ("geometric", mean) | ("uniform", lo, hi) | ("fixed", doc_ids array)
            | ("single",) (one document)
    c_kind: "normal0.5"  C ~ N(0, 0.5^2), mixed signs
            "onehot80"   per token: with prob 0.8 C[t,:] = e_h, h ~ U{0..H-1},
                         else N(0, 0.5^2)
            "normal1neg" C ~ N(0, 1), then a seeded 10% of entries -> -U(4, 8)
    g_kind: "u0.5-1.5" | "one" | "u0-2"
    """
    assert dtype in ("bf16", "f32")
    rng = np.random.default_rng(seed)
    kind = docs[0]
    if kind == "geometric":
        doc = geometric_docs(rng, T, docs[1])
    elif kind == "uniform":
        doc = uniform_docs(rng, T, docs[1], docs[2])
    elif kind == "fixed":
        doc = np.ascontiguousarray(docs[1], dtype=np.int32)
        assert doc.shape == (T,)
    elif kind == "single":
        doc = np.zeros(T, dtype=np.int32)
    else:
        raise ValueError(kind)

    rnd = round_bf16 if dtype == "bf16" else (lambda x: x)
    q = _normal(rng, (T, H, d))
    k = _normal(rng, (T, H, d))
    if qk_rms:
        q, k = _rms_rows(q), _rms_rows(k)
    q, k = rnd(q), rnd(k)
    v = rnd(_normal(rng, (T, H, d)))

    if c_kind == "normal0.5":
        c = (0.5 * _normal(rng, (T, H))).astype(np.float32)
    elif c_kind == "onehot80":
        u = rng.random(T)
        hsel = rng.integers(0, H, size=T)
        c = (0.5 * _normal(rng, (T, H))).astype(np.float32)
        onehot = u < 0.8
        c[onehot] = 0.0
        c[np.nonzero(onehot)[0], hsel[onehot]] = 1.0
    elif c_kind == "normal1neg":
        c = _normal(rng, (T, H))
        sel = rng.random((T, H)) < 0.10
        c[sel] = -rng.uniform(4.0, 8.0, size=int(sel.sum())).astype(np.float32)
    else:
        raise ValueError(c_kind)

    if g_kind == "u0.5-1.5":
        g = rng.uniform(0.5, 1.5, size=(T, H)).astype(np.float32)
    elif g_kind == "one":
        g = np.ones((T, H), dtype=np.float32)
    elif g_kind == "u0-2":
        g = rng.uniform(0.0, 2.0, size=(T, H)).astype(np.float32)
    else:
        raise ValueError(g_kind)

    do = rnd(_normal(rng, (T, H, d))) if with_do else None
    return Workload(name=name or f"T{T}_H{H}_d{d}_{dtype}_s{seed}", T=T, H=H, d=d,
                    window=window, dtype=dtype,
                    scale=(1.0 / math.sqrt(d)) if scale is None else float(scale),
                    q=q, k=k, v=v, c=c, g=g, doc=doc, do=do,
                    recipe=f"docs={docs[0]}{tuple(docs[1:]) if kind != 'fixed' else ''} "
                           f"qk_rms={qk_rms} C={c_kind} G={g_kind} seed={seed}")


# The five reference workloads.  Index 1 is the GPT-2 small layer forward the
# throughput figure is quoted on; index 2 is the same layer forward+backward.
CONFIGS = {
    0: dict(T=256, H=2, d=16, dtype="f32", seed=0,
            docs=("fixed", np.array([0] * 100 + [1] * 156, dtype=np.int32)),
            qk_rms=False, c_kind="normal0.5", g_kind="u0.5-1.5",
            name="tiny_f32_T256_H2_d16", passes="fwd"),
    1: dict(T=65536, H=6, d=128, dtype="bf16", seed=1, docs=("geometric", 1024),
            qk_rms=True, c_kind="normal0.5", g_kind="u0.5-1.5",
            name="gpt2s_fwd_T65536_H6_d128", passes="fwd"),
    2: dict(T=65536, H=6, d=128, dtype="bf16", seed=2, docs=("geometric", 1024),
            qk_rms=True, c_kind="normal0.5", g_kind="u0.5-1.5",
            name="gpt2s_fwdbwd_T65536_H6_d128", passes="fwd+bwd"),
    3: dict(T=131072, H=12, d=64, dtype="bf16", seed=3, docs=("geometric", 2048),
            qk_rms=True, c_kind="onehot80", g_kind="one",
            name="wide_fwdbwd_T131072_H12_d64", passes="fwd+bwd"),
    4: dict(T=262144, H=6, d=128, dtype="bf16", seed=4, docs=("uniform", 8, 256),
            qk_rms=True, c_kind="normal1neg", g_kind="u0-2",
            name="stress_fwdbwd_T262144_H6_d128", passes="fwd+bwd"),
}


def config_workload(i: int, T: Optional[int] = None) -> Workload:
    """Workload i of the five reference configurations.  `T` truncates the
    stream (same draws for the document lengths, fewer tokens) for quick runs."""
    cfg = dict(CONFIGS[i])
    cfg.pop("passes")
    if T is not None and T != cfg["T"]:
        cfg["T"] = T
        if cfg["docs"][0] == "fixed":
            cfg["docs"] = ("fixed", cfg["docs"][1][:T])
        cfg["name"] = cfg["name"] + f"_trunc{T}"
    return make_workload(**cfg)



# ----------------------------------------------------------------------------
# Full DCMHA composition (AITNT page, section "第二刀-砍层内", DCMHA paragraph)
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class DcmhaWorkload:
    name: str
    T: int
    H: int
    d: int
    window: int
    dtype: str
    scale: float
    q: np.ndarray       # [T, H, d] float32 (values representable in `dtype`)
    k: np.ndarray
    v: np.ndarray
    cs: np.ndarray      # [T, H, H] float32 score composition
    cw: np.ndarray      # [T, H, H] float32 weight composition
    doc: np.ndarray     # [T] int32
    do: np.ndarray      # [T, H, d] float32 (representable in `dtype`)
    recipe: str = ""

    def torch_inputs(self, device="cuda"):
        import torch

        def big(x):
            if self.dtype == "bf16":
                return torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(device)
            return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)

        f = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(device)
        return dict(q=big(self.q), k=big(self.k), v=big(self.v), cs=f(self.cs), cw=f(self.cw),
                    doc=f(self.doc), do=big(self.do))


def _composition(rng, kind: str, T: int, H: int) -> np.ndarray:
    """[T, H, H] per-query head compositions.
    "eye+normal0.3": I + N(0, 0.3^2) (each head keeps mostly its own map, mixed
                     with every other head's, either sign);
    "eye":           the identity;
    "perm":          a random permutation matrix per query."""
    if kind == "eye+normal0.3":
        return (np.eye(H, dtype=np.float32)[None] + 0.3 * _normal(rng, (T, H, H))).astype(np.float32)
    if kind == "eye":
        return np.broadcast_to(np.eye(H, dtype=np.float32)[None], (T, H, H)).copy()
    if kind == "perm":
        out = np.zeros((T, H, H), dtype=np.float32)
        for t in range(T):
            out[t, np.arange(H), rng.permutation(H)] = 1.0
        return out
    raise ValueError(kind)


def make_dcmha_workload(T: int, H: int, d: int, *, window: int = WINDOW, dtype: str = "bf16",
                        seed: int = 0, docs=("geometric", 1024), qk_rms: bool = True,
                        cs_kind: str = "eye+normal0.3", cw_kind: str = "eye+normal0.3",
                        scale: Optional[float] = None, name: Optional[str] = None) -> DcmhaWorkload:
    """Seeded DCMHA workload.  Draw order (one PCG64 stream): document lengths,
    Q, K, V, CS, CW, dO; Q, K, V, dO rounded to bf16 (RNE) for bf16 workloads.
    cs_kind / cw_kind as in _composition; cw_kind "ldc" takes G[t,h] C[t,:]
    with C ~ N(0, 0.5^2), G ~ U(0.5, 1.5) (the Lightweight DC layer's weights,
    drawn C then G)."""
    assert dtype in ("bf16", "f32")
    rng = np.random.default_rng(seed)
    kind = docs[0]
    if kind == "geometric":
        doc = geometric_docs(rng, T, docs[1])
    elif kind == "uniform":
        doc = uniform_docs(rng, T, docs[1], docs[2])
    elif kind == "single":
        doc = np.zeros(T, dtype=np.int32)
    else:
        raise ValueError(kind)
    rnd = round_bf16 if dtype == "bf16" else (lambda x: x)
    q = _normal(rng, (T, H, d))
    k = _normal(rng, (T, H, d))
    if qk_rms:
        q, k = _rms_rows(q), _rms_rows(k)
    q, k = rnd(q), rnd(k)
    v = rnd(_normal(rng, (T, H, d)))
    cs = _composition(rng, cs_kind, T, H)
    if cw_kind == "ldc":
        c = (0.5 * _normal(rng, (T, H))).astype(np.float32)
        g = rng.uniform(0.5, 1.5, size=(T, H)).astype(np.float32)
        cw = (g[:, :, None] * c[:, None, :]).astype(np.float32)
    else:
        cw = _composition(rng, cw_kind, T, H)
    do = rnd(_normal(rng, (T, H, d)))
    return DcmhaWorkload(name=name or f"dcmha_T{T}_H{H}_d{d}_{dtype}_s{seed}", T=T, H=H, d=d,
                         window=window, dtype=dtype,
                         scale=(1.0 / math.sqrt(d)) if scale is None else float(scale),
                         q=q, k=k, v=v, cs=cs, cw=cw, doc=doc, do=do,
                         recipe=f"docs={docs[0]}{tuple(docs[1:])} qk_rms={qk_rms} CS={cs_kind} "
                                f"CW={cw_kind} seed={seed}")


# The DCMHA benchmark workload: the GPT-2 small attention shape of the
# Lightweight DC configurations, forward+backward.
DCMHA_BENCH = dict(T=65536, H=6, d=128, dtype="bf16", seed=5, docs=("geometric", 1024),
                   cs_kind="eye+normal0.3", cw_kind="eye+normal0.3",
                   name="dcmha_gpt2s_fwdbwd_T65536_H6_d128")


# ----------------------------------------------------------------------------
# Generator of the Lightweight DC weights (C = x WC, G = x WG)
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class CgWorkload:
    name: str
    T: int
    dm: int
    H: int
    dtype: str
    x: np.ndarray       # [T, dm] float32 (representable in `dtype`)
    wc: np.ndarray      # [dm, H]
    wg: np.ndarray      # [dm, H]
    dc: np.ndarray      # [T, H] float32
    dg: np.ndarray      # [T, H] float32
    recipe: str = ""

    def torch_inputs(self, device="cuda"):
        import torch

        def big(a):
            if self.dtype == "bf16":
                return torch.from_numpy(bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(device)
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

        f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return dict(x=big(self.x), wc=big(self.wc), wg=big(self.wg), dc=f(self.dc), dg=f(self.dg))


def make_cg_workload(T: int, dm: int, H: int, *, dtype: str = "bf16", seed: int = 0,
                     name: Optional[str] = None) -> CgWorkload:
    """Seeded generator workload.  Draw order: x, WC, WG, dC, dG.  x rows are
    RMS-normalised N(0, 1) (a normalised hidden state); WC ~ N(0, 0.5^2/dm)
    so that C ~ N(0, 0.5^2) like the Lightweight DC recipe's C; WG ~ N(0, 1/dm);
    dC, dG ~ N(0, 1).  x, WC, WG rounded to bf16 for bf16 workloads."""
    assert dtype in ("bf16", "f32")
    rng = np.random.default_rng(seed)
    rnd = round_bf16 if dtype == "bf16" else (lambda a: a)
    x = rnd(_rms_rows(_normal(rng, (T, dm))))
    wc = rnd((0.5 / math.sqrt(dm) * _normal(rng, (dm, H))).astype(np.float32))
    wg = rnd((1.0 / math.sqrt(dm) * _normal(rng, (dm, H))).astype(np.float32))
    dc = _normal(rng, (T, H))
    dg = _normal(rng, (T, H))
    return CgWorkload(name=name or f"cg_T{T}_dm{dm}_H{H}_{dtype}_s{seed}", T=T, dm=dm, H=H, dtype=dtype,
                      x=x, wc=wc, wg=wg, dc=dc, dg=dg,
                      recipe=f"x=rms(N(0,1)) WC=N(0,0.25/dm) WG=N(0,1/dm) dC,dG=N(0,1) seed={seed}")


# The generator's benchmark workload: the GPT-2 small hidden state feeding
# the 6-head layer (model dim 768).
CG_BENCH = dict(T=65536, dm=768, H=6, dtype="bf16", seed=6, name="cg_gpt2s_T65536_dm768_H6")


# ----------------------------------------------------------------------------
# MUDD layer mixing (AITNT page, section "第一刀—砍层间")
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class MuddWorkload:
    """Inputs of a MUDD mix: J layer streams X_j [T, dm], weights A [T, W, J]
    and the upstream gradients dY_w [T, dm] of the W ways."""
    name: str
    T: int
    dm: int
    W: int
    J: int
    dtype: str          # storage type of the streams and of dY
    xs: list            # J arrays [T, dm] float32 (representable in `dtype`)
    a: np.ndarray       # [T, W, J] float32
    dys: list           # W arrays [T, dm] float32 (representable in `dtype`)
    recipe: str = ""

    def slice(self, lo: int, hi: int) -> "MuddWorkload":
        return dataclasses.replace(self, name=f"{self.name}[{lo}:{hi}]", T=hi - lo,
                                   xs=[x[lo:hi] for x in self.xs], a=self.a[lo:hi],
                                   dys=[d[lo:hi] for d in self.dys])

    def torch_inputs(self, device="cuda"):
        """(xs, a, dys) as torch tensors on `device`, streams in the storage dtype."""
        import torch

        def big(x):
            if self.dtype == "bf16":
                return torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(device)
            return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)

        return ([big(x) for x in self.xs],
                torch.from_numpy(np.ascontiguousarray(self.a)).to(device),
                [big(d) for d in self.dys])


def make_mudd_workload(T: int, dm: int, W: int, J: int, *, dtype: str = "bf16", seed: int = 0,
                       a_std: float = 0.5, name: Optional[str] = None) -> MuddWorkload:
    """Seeded MUDD inputs.  Draw order (one PCG64 stream): X_0 .. X_{J-1}
    ~ N(0, 1), A ~ N(0, a_std^2) (weights of both signs, as the page allows),
    dY_0 .. dY_{W-1} ~ N(0, 1); streams and dY rounded to bf16 (RNE) for
    bf16 workloads."""
    if dtype not in ("bf16", "f32"):
        raise ValueError("dtype must be 'bf16' or 'f32'")
    rng = np.random.default_rng(seed)
    rnd = round_bf16 if dtype == "bf16" else (lambda x: x)
    xs = [rnd(_normal(rng, (T, dm))) for _ in range(J)]
    a = (_normal(rng, (T, W, J)) * np.float32(a_std)).astype(np.float32)
    dys = [rnd(_normal(rng, (T, dm))) for _ in range(W)]
    nm = name or f"mudd_T{T}_dm{dm}_W{W}_J{J}_{dtype}"
    recipe = (f"T={T} tokens, dm={dm}, {W} way(s), {J} streams, {dtype}; X, dY ~ N(0,1), "
              f"A ~ N(0,{a_std}^2), seed {seed}")
    return MuddWorkload(nm, T, dm, W, J, dtype, xs, a, dys, recipe)


# The mixing workload the benchmark times: a GPT-2 small stream (65,536 tokens,
# model_dim 768) at the widest point of a 12-layer model (embedding plus 12
# layer outputs) with the four ways of full MUDD.
MUDD_BENCH = dict(T=65536, dm=768, W=4, J=13, dtype="bf16", seed=11)
