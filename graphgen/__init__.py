"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module only *draws inputs*: graphs (as CSR) and feature tensors.  It holds none of
the attention arithmetic, so the oracle and the HIP path can both consume its arrays
without sharing any computation.

Graph families follow the workloads used to evaluate fused graph attention: an
Erdos-Renyi digraph, Chung-Lu power-law graphs and an R-MAT graph.  The pages that
describe the method ("On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
Technical Summary > Results) evaluate on OGB, citation and GraphLand graphs, none of
which is available here; these generators stand in for them with the stated shapes,
degree distributions and sizes.

Conventions
-----------
* One RNG per (workload id, stream): ``np.random.default_rng(SeedSequence([wid, stream]))``
  with stream 0 = graph, 1 = features, 2 = upstream gradient.
* CSR row i is a *destination*; ``indices[indptr[i]:indptr[i+1]]`` are its sources,
  ascending.  Sampled self-loops are dropped, then exactly one (i, i) edge is added per
  node.  Parallel edges are kept (each CSR entry is one edge).
* Node ids are relabelled by a seeded random permutation so that ids carry no degree
  information.
* bf16 tensors are carried as ``np.uint16`` bit patterns, produced from fp32 draws by
  round-to-nearest-even.
"""
from __future__ import annotations

import hashlib
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "rng_for", "erdos_renyi_edges", "chung_lu_edges", "chung_lu_offset", "rmat_edges",
    "finish_csr", "csr_from_edges", "random_multigraph", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "normal_features", "Workload", "WORKLOADS", "make_graph",
    "make_features", "make_dout", "array_digest",
]


def rng_for(wid: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(wid), int(stream)]))


# ----------------------------------------------------------------------------- graphs

def erdos_renyi_edges(n: int, p: float, rng: np.random.Generator):
    """Directed G(n, p): an independent Bernoulli(p) for every ordered pair i != j.

    Returns (src, dst) int64 arrays.  Row-major over (dst, src) so the draw order is fixed.
    """
    src_l, dst_l = [], []
    block = max(1, (1 << 22) // max(n, 1))
    for d0 in range(0, n, block):
        d1 = min(n, d0 + block)
        hit = rng.random((d1 - d0, n)) < p
        hit[np.arange(d1 - d0), np.arange(d0, d1)] = False
        dd, ss = np.nonzero(hit)
        dst_l.append(dd.astype(np.int64) + d0)
        src_l.append(ss.astype(np.int64))
    return np.concatenate(src_l), np.concatenate(dst_l)


def chung_lu_offset(n: int, gamma: float, max_over_mean: float, iters: int = 200) -> float:
    """Offset i0 so that w_i = (i + i0)^(-1/(gamma-1)) has max(w)/mean(w) == max_over_mean.

    Fixed-count bisection (the ratio falls monotonically as i0 grows).
    """
    beta = 1.0 / (gamma - 1.0)
    idx = np.arange(n, dtype=np.float64)

    def ratio(i0):
        w = (idx + i0) ** (-beta)
        return w[0] / w.mean()

    lo, hi = 1e-9, float(n)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if ratio(mid) > max_over_mean:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def chung_lu_edges(n: int, m: int, gamma: float, max_over_mean: float, rng: np.random.Generator):
    """Chung-Lu multigraph: m edges whose src and dst are drawn independently with
    P(v) ~ w_v.  Parallel edges are kept.  Returns (src, dst) int64.

    Sampled as per-node counts: dst counts ~ Multinomial(m, p) laid out in node order,
    src counts ~ Multinomial(m, p) laid out then shuffled by a uniform permutation.  The
    pairs are i.i.d. (dst, src) draws, as with per-edge sampling, at O(n + m) cost.
    """
    i0 = chung_lu_offset(n, gamma, max_over_mean)
    w = (np.arange(n, dtype=np.float64) + i0) ** (-1.0 / (gamma - 1.0))
    p = w / w.sum()
    nodes = np.arange(n, dtype=np.int64)
    dst = np.repeat(nodes, rng.multinomial(m, p))
    src = np.repeat(nodes, rng.multinomial(m, p))
    src = src[rng.permutation(m)]
    return src, dst


def rmat_edges(scale: int, m: int, a: float, b: float, c: float, rng: np.random.Generator,
               chunk: int = 1 << 23):
    """R-MAT edge list: for each edge and each of ``scale`` bit levels (MSB first), pick a
    quadrant with probabilities (a, b, c, 1-a-b-c) = (src0/dst0, src0/dst1, src1/dst0,
    src1/dst1).  No noise; parallel edges kept.  Returns (src, dst) int64.
    """
    src = np.zeros(m, dtype=np.int64)
    dst = np.zeros(m, dtype=np.int64)
    ab, abc = a + b, a + b + c
    for s0 in range(0, m, chunk):
        s1 = min(m, s0 + chunk)
        sv = src[s0:s1]
        dv = dst[s0:s1]
        for _ in range(scale):
            r = rng.random(s1 - s0)
            sbit = r >= ab
            dbit = ((r >= a) & (r < ab)) | (r >= abc)
            sv <<= 1
            dv <<= 1
            sv += sbit
            dv += dbit
    return src, dst


def finish_csr(n: int, src: np.ndarray, dst: np.ndarray, rng: np.random.Generator | None,
               relabel: bool = True, self_loops: bool = True):
    """Relabel ids (seeded permutation), drop sampled self-loops, add one (i, i) per node,
    and build CSR (row = dst) with sources ascending within each row.
    Returns (indptr int32 [n+1], indices int32 [E]).
    """
    if relabel:
        perm = rng.permutation(n).astype(np.int64)
        src = perm[src]
        dst = perm[dst]
    if self_loops:
        keep = src != dst
        src = src[keep]
        dst = dst[keep]
        loops = np.arange(n, dtype=np.int64)
        src = np.concatenate([src, loops])
        dst = np.concatenate([dst, loops])
    key = dst.astype(np.int64) * np.int64(n) + src.astype(np.int64)
    del src, dst
    key.sort(kind="stable")
    counts = np.bincount(key // n, minlength=n) if n > 0 else np.zeros(0, np.int64)
    indptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(counts, out=indptr[1:])
    if indptr[-1] >= 2 ** 31:
        raise ValueError("edge count does not fit int32")
    indices = (key % n).astype(np.int32) if n > 0 else np.zeros(0, np.int32)
    return indptr.astype(np.int32), indices


def csr_from_edges(n: int, src, dst):
    """CSR (row = dst) of an explicit edge list, keeping parallel edges, no relabel."""
    src = np.asarray(src, dtype=np.int64)
    dst = np.asarray(dst, dtype=np.int64)
    return finish_csr(n, src, dst, None, relabel=False, self_loops=False)


def random_multigraph(n: int, m: int, rng: np.random.Generator, self_loops=True,
                      hub_rows=(), hub_deg=0):
    """Small uniform multigraph (parallel edges likely when m ~ n^2) with optional hub rows
    that receive ``hub_deg`` extra in-edges each.  For tests."""
    src = rng.integers(0, n, m)
    dst = rng.integers(0, n, m)
    for h in hub_rows:
        src = np.concatenate([src, rng.integers(0, n, hub_deg)])
        dst = np.concatenate([dst, np.full(hub_deg, h)])
    return finish_csr(n, src, dst, rng, relabel=False, self_loops=self_loops)


# --------------------------------------------------------------------------- features

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) by round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_features(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


# -------------------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    graph: str                 # "er" | "chunglu" | "rmat"
    n: int
    heads: int
    dim: int
    dtype: str                 # "f32" | "bf16"
    score: str                 # "dot" | "gat" | "gatv2" | "max" | "min" (reductions)
    backward: bool
    graph_args: dict = field(default_factory=dict)
    graph_wid: int = 0         # wid whose graph/feature streams this workload reuses (0 = own)

    @property
    def seed_id(self) -> int:
        return self.graph_wid or self.wid


WORKLOADS = {
    w.name: w for w in [
        Workload(1, "er2k_dot_f32", "er", 2000, 1, 32, "f32", "dot", False,
                 {"p": 8.0 / 1999.0}),
        Workload(2, "chunglu100k_gat_f32", "chunglu", 100_000, 4, 64, "f32", "gat", False,
                 {"avg_deg": 20, "gamma": 2.1, "max_over_mean": 500.0}),
        Workload(3, "chunglu1m_dot_bf16", "chunglu", 1_000_000, 8, 32, "bf16", "dot", False,
                 {"avg_deg": 50, "gamma": 2.1, "max_over_mean": 500.0}),
        Workload(4, "rmat21_dot_bf16", "rmat", 1 << 21, 1, 128, "bf16", "dot", False,
                 {"scale": 21, "avg_deg": 30, "a": 0.57, "b": 0.19, "c": 0.19}),
        Workload(5, "chunglu1m_train_bf16", "chunglu", 1_000_000, 8, 32, "bf16", "dot", True,
                 {"avg_deg": 50, "gamma": 2.1, "max_over_mean": 500.0}, graph_wid=3),
        Workload(6, "chunglu1m_gatv2_train_bf16", "chunglu", 1_000_000, 8, 32, "bf16", "gatv2",
                 True, {"avg_deg": 50, "gamma": 2.1, "max_over_mean": 500.0}, graph_wid=3),
        Workload(7, "chunglu1m_max_train_bf16", "chunglu", 1_000_000, 8, 32, "bf16", "max",
                 True, {"avg_deg": 50, "gamma": 2.1, "max_over_mean": 500.0}, graph_wid=3),
        Workload(8, "chunglu100k_gat_train_f32", "chunglu", 100_000, 4, 64, "f32", "gat", True,
                 {"avg_deg": 20, "gamma": 2.1, "max_over_mean": 500.0}, graph_wid=2),
    ]
}


def _cached(tag: str, build):
    """Memoise ``build()`` (a tuple of arrays) as .npy files under $GRAPHGEN_CACHE, if set."""
    root = os.environ.get("GRAPHGEN_CACHE")
    if not root:
        return build()
    os.makedirs(root, exist_ok=True)
    base = os.path.join(root, tag)
    done = base + ".done"
    if os.path.exists(done):
        k = int(open(done).read())
        return tuple(np.load(f"{base}.{i}.npy", allow_pickle=False) for i in range(k))
    out = build()
    for i, a in enumerate(out):
        np.save(f"{base}.{i}.npy", a, allow_pickle=False)
    with open(done, "w") as f:
        f.write(str(len(out)))
    return out


def make_graph(w: Workload, n: int | None = None):
    """CSR of workload ``w``; ``n`` overrides the node count (same recipe, fewer nodes)."""
    n = w.n if n is None else int(n)
    return _cached(f"graph_{w.seed_id}_{n}", lambda: _make_graph(w, n))


def _make_graph(w: Workload, n: int):
    rng = rng_for(w.seed_id, 0)
    ga = w.graph_args
    if w.graph == "er":
        p = ga["p"] if n == w.n else 8.0 / max(n - 1, 1)
        src, dst = erdos_renyi_edges(n, p, rng)
    elif w.graph == "chunglu":
        src, dst = chung_lu_edges(n, ga["avg_deg"] * n, ga["gamma"], ga["max_over_mean"], rng)
    elif w.graph == "rmat":
        scale = ga["scale"] if n == w.n else int(np.log2(n))
        if (1 << scale) != n:
            raise ValueError("R-MAT needs a power-of-two node count")
        src, dst = rmat_edges(scale, ga["avg_deg"] * n, ga["a"], ga["b"], ga["c"], rng)
    else:
        raise ValueError(w.graph)
    return finish_csr(n, src, dst, rng)


def make_features(w: Workload, n: int | None = None):
    """Inputs of the forward pass, drawn in a fixed order from the feature stream.

    dot: (q, k, v) each [n, H, d];  gat: (s [n, H] f32, t [n, H] f32, v [n, H, d]);
    gatv2: (xd [n, H, d], xs [n, H, d], attn [H, d] f32 ~ N(0, 1/d));
    max / min: (x [n, H, d],) (the first draw of the stream, like q).
    """
    n = w.n if n is None else int(n)
    tag = {"gatv2": "_gatv2", "max": "_red", "min": "_red"}.get(w.score, "")
    return _cached(f"feat{tag}_{w.seed_id}_{n}", lambda: _make_features(w, n))


def _make_features(w: Workload, n: int):
    rng = rng_for(w.seed_id, 1)
    H, d = w.heads, w.dim
    if w.score == "dot":
        q = normal_features(rng, (n, H, d), w.dtype)
        k = normal_features(rng, (n, H, d), w.dtype)
        v = normal_features(rng, (n, H, d), w.dtype)
        return q, k, v
    if w.score in ("max", "min"):
        return (normal_features(rng, (n, H, d), w.dtype),)
    if w.score == "gatv2":
        xd = normal_features(rng, (n, H, d), w.dtype)
        xs = normal_features(rng, (n, H, d), w.dtype)
        attn = (rng.standard_normal(size=(H, d), dtype=np.float32) / np.float32(np.sqrt(d)))
        return xd, xs, attn.astype(np.float32)
    s = rng.standard_normal(size=(n, H), dtype=np.float32)
    t = rng.standard_normal(size=(n, H), dtype=np.float32)
    v = normal_features(rng, (n, H, d), w.dtype)
    return s, t, v


def make_dout(w: Workload, n: int | None = None):
    n = w.n if n is None else int(n)
    return _cached(f"dout_{w.seed_id}_{n}",
                   lambda: (normal_features(rng_for(w.seed_id, 2), (n, w.heads, w.dim),
                                            w.dtype),))[0]


def array_digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode())
        h.update(str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()
