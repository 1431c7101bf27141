"""Seeded synthetic workloads for the MoE forward path.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no routing, sorting, matrix products or combine).
Both the HIP path and the CPU oracle consume the arrays it returns, so the
two sides always see bit-identical inputs.

Every tensor comes from its own numpy ``Generator(PCG64(SeedSequence(
[1000 + cfg.index, stream, index])))``:

  stream 1 logits, 2 x, 3 w13 (index = expert), 4 w2 (index = expert),
  5 shared w13, 6 shared w2, 7 cold-expert split of the EP share,
  8 gates of the EP share, 9 parity sample, 10 router matrix.

Normal draws are fp32 ``standard_normal`` times the stated std; bf16
tensors are those fp32 draws rounded to nearest-even and kept as uint16 bit
patterns (numpy has no bf16 type).

The five workloads are the shapes the pages discuss: a small fp32 layer
(1,024 tokens, 8 experts over 4 ranks, the study guide's worked example in
"Expert Parallelism at Scale", section "Worked example"), a Mixtral-8x7B
layer, DeepSeek-V3 decode and prefill layers, and one GPU's share of
64-way expert parallelism with a 50% hot expert.
"""
from __future__ import annotations

import os
import sys
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

S_LOGITS, S_X, S_W13, S_W2, S_SH_W13, S_SH_W2, S_COLD, S_GATES, S_SAMPLE, S_ROUTER = range(1, 11)


@dataclass(frozen=True)
class MoeConfig:
    name: str
    index: int              # 1..5; the seed root is 1000 + index
    T: int                  # tokens (for the EP share: received rows)
    E: int                  # experts held on this GPU
    k: int                  # assignments per token
    d: int                  # model width
    ffn: int                # expert hidden width
    dtype: str              # "f32" or "bf16"
    gating: str             # "softmax", "sigmoid" or "given" (EP share: ids and gates are inputs)
    renormalize: int = 1
    n_groups: int = 1
    topk_groups: int = 1
    shared: bool = False    # one always-active shared expert of width ffn
    n_ep: int = 0           # simulated expert-parallel group for the send-count matrix (0: none)
    w_std: float = 0.02
    n_src: int = 0          # EP share: number of simulated source ranks
    note: str = field(default="", compare=False)

    @property
    def M(self) -> int:
        return self.T * self.k

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS = {
    "small_fp32": MoeConfig(
        "small_fp32", 1, T=1024, E=8, k=2, d=256, ffn=512, dtype="f32",
        gating="softmax", renormalize=1, n_ep=4,
        note="4 simulated ranks x 256 tokens, 2 experts per rank, top-2 softmax"),
    "mixtral_bf16": MoeConfig(
        "mixtral_bf16", 2, T=4096, E=8, k=2, d=4096, ffn=14336, dtype="bf16",
        gating="softmax", renormalize=1,
        note="Mixtral-8x7B shape, top-2 softmax renormalised over the chosen 2"),
    "dsv3_decode": MoeConfig(
        "dsv3_decode", 3, T=128, E=256, k=8, d=7168, ffn=2048, dtype="bf16",
        gating="sigmoid", renormalize=1, shared=True,
        note="DeepSeek-V3 decode batch, ~4 rows per expert, plain top-8"),
    "dsv3_prefill": MoeConfig(
        "dsv3_prefill", 4, T=8192, E=256, k=8, d=7168, ffn=2048, dtype="bf16",
        gating="sigmoid", renormalize=1, n_groups=8, topk_groups=4, shared=True, n_ep=64,
        note="DeepSeek-V3 prefill, 8 groups of 32, top-4 groups, top-8"),
    "ep64_share": MoeConfig(
        "ep64_share", 5, T=32768, E=4, k=1, d=7168, ffn=2048, dtype="bf16",
        gating="given", renormalize=0, n_src=64,
        note="one GPU of EP=64: 4 local experts, 64 sources x 512 rows, hot expert 0 takes 50%"),
}
CONFIG_ORDER = ["small_fp32", "mixtral_bf16", "dsv3_decode", "dsv3_prefill", "ep64_share"]


def rng(cfg: MoeConfig, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + cfg.index, stream, index])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(g: np.random.Generator, n: int, std: float, dtype: str) -> np.ndarray:
    a = g.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a if dtype == "f32" else f32_to_bf16_bits(a)


class _Scratch(threading.local):
    f32 = None
    u32 = None


_scratch = _Scratch()


def _normal_into(out: np.ndarray, g: np.random.Generator, std: float) -> None:
    """Fill out (fp32, or uint16 bf16 bits) with N(0, std) draws.  Identical values
    to _normal(); reuses per-thread scratch so no fresh pages are touched per call."""
    n = out.size
    flat = out.reshape(-1)
    if out.dtype == np.float32:
        g.standard_normal(n, dtype=np.float32, out=flat)
        if std != 1.0:
            flat *= np.float32(std)
        return
    if _scratch.f32 is None or _scratch.f32.size < n:
        _scratch.f32 = np.empty(n, np.float32)
        _scratch.u32 = np.empty(n, np.uint32)
    a = _scratch.f32[:n]
    g.standard_normal(n, dtype=np.float32, out=a)
    if std != 1.0:
        a *= np.float32(std)
    u = a.view(np.uint32)
    t = _scratch.u32[:n]
    np.right_shift(u, np.uint32(16), out=t)          # round to nearest even:
    np.bitwise_and(t, np.uint32(1), out=t)           # u + 0x7FFF + lsb(u >> 16)
    np.add(t, np.uint32(0x7FFF), out=t)
    np.add(t, u, out=t)
    np.right_shift(t, np.uint32(16), out=t)
    np.copyto(flat, t, casting="unsafe")


def gen_logits(cfg: MoeConfig) -> np.ndarray:
    """Router logits [T, E], fp32 N(0,1)."""
    return rng(cfg, S_LOGITS).standard_normal((cfg.T, cfg.E), dtype=np.float32)


def gen_router_weights(cfg: MoeConfig) -> np.ndarray:
    """Router matrix [E, d], N(0, 1/d) in the layer dtype, so that with x ~ N(0,1)
    the router's logits are ~N(0,1) like gen_logits'."""
    return _normal(rng(cfg, S_ROUTER), cfg.E * cfg.d, 1.0 / np.sqrt(cfg.d), cfg.dtype).reshape(cfg.E, cfg.d)


def gen_x(cfg: MoeConfig) -> np.ndarray:
    """Token activations [T, d] (EP share: received rows), N(0,1); fp32 or bf16 bits."""
    return _normal(rng(cfg, S_X), cfg.T * cfg.d, 1.0, cfg.dtype).reshape(cfg.T, cfg.d)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def gen_expert_weights(cfg: MoeConfig, experts=None, shared: bool = False, verbose: bool = False):
    """Expert weights, N(0, w_std).

    w13 [G, 2, ffn, d]: per expert the gate matrix then the up matrix, each row
    an output feature with its d inputs contiguous.  w2 [G, d, ffn]: the down
    matrix, each row a model feature with its ffn inputs contiguous.
    ``experts`` selects routed experts (default: all); ``shared`` returns the one
    shared expert instead (G = 1).
    """
    if shared:
        ids, s13, s2 = [0], S_SH_W13, S_SH_W2
    else:
        ids, s13, s2 = (list(range(cfg.E)) if experts is None else list(experts)), S_W13, S_W2
    G, d, ffn = len(ids), cfg.d, cfg.ffn
    wdt = np.float32 if cfg.dtype == "f32" else np.uint16
    w13 = np.empty((G, 2, ffn, d), dtype=wdt)
    w2 = np.empty((G, d, ffn), dtype=wdt)

    def one(i):
        e = ids[i]
        _normal_into(w13[i], rng(cfg, s13, e), cfg.w_std)
        _normal_into(w2[i], rng(cfg, s2, e), cfg.w_std)
        if verbose and (i + 1) % 32 == 0:
            print(f"  weights: {i + 1}/{G} experts", file=sys.stderr, flush=True)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(G)))
    return w13, w2


def gen_ep_share_routing(cfg: MoeConfig):
    """Received-row expert ids and gates for one GPU's EP share.

    ``n_src`` source ranks each send T/n_src rows, source-major.  Each source's
    block is already in local-expert order (the sender sorted it): half of the
    block goes to hot expert 0, the other half is split over experts 1..E-1 by a
    seeded uniform multinomial.  Gates are U(0,1) fp32.  Returns ids [T,1] int32
    and gates [T,1] fp32.
    """
    per = cfg.T // cfg.n_src
    hot = per // 2
    g = rng(cfg, S_COLD)
    blocks = []
    for _ in range(cfg.n_src):
        cold = g.multinomial(per - hot, [1.0 / (cfg.E - 1)] * (cfg.E - 1))
        blk = np.concatenate([np.zeros(hot, np.int32)] +
                             [np.full(c, e + 1, np.int32) for e, c in enumerate(cold)])
        blocks.append(blk)
    ids = np.concatenate(blocks).reshape(cfg.T, 1)
    gates = rng(cfg, S_GATES).random(cfg.T, dtype=np.float32).reshape(cfg.T, 1)
    return ids, gates


def sample_tokens(cfg: MoeConfig, n: int = 256) -> np.ndarray:
    """A seeded, sorted sample of n distinct token (row) indices for sampled parity."""
    n = min(n, cfg.T)
    return np.sort(rng(cfg, S_SAMPLE).choice(cfg.T, size=n, replace=False)).astype(np.int64)
