"""Seeded input generators.

Every random tensor comes from NumPy's PCG64 stream keyed by
SeedSequence([seed, config id, tensor id, layer]), so any tensor of any config can be
regenerated alone. bf16 tensors are returned as uint16 bit patterns (NumPy has no
bf16 dtype); the bindings reinterpret them as torch.bfloat16.

Large bench-scale tensors can instead be drawn directly on the GPU with
`torch_normal_bf16`, which uses torch's device generator with the same seed key.
That stream differs from the NumPy one; it serves timing only, where no oracle
comparison is made of the whole tensor.
"""

import numpy as np

# Tensor ids of the seed key.
TID_W = 1            # linear weights: layer * 16 + slot
TID_X = 2            # linear-layer activations
TID_Q = 3            # attention queries
TID_KC = 4           # prefix K cache
TID_VC = 5           # prefix V cache
TID_KT = 6           # tree K
TID_VT = 7           # tree V
TID_TREE = 8         # tree shape
TID_TOK = 9          # tree tokens
TID_LOGIT = 10       # seeded target logits
TID_GUMBEL = 11      # Gumbel noise
TID_NORM = 12        # RMSNorm gains
TID_EMBED = 13       # embedding table
TID_LMHEAD = 14      # LM head
TID_HIDDEN = 15      # hidden-state inputs

SLOT = {"qkv": 0, "o": 1, "gate_up": 2, "down": 3}


def rng(seed: int, cid: int, tid: int, layer: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cid, tid, layer]))


def bf16_bits(x) -> np.ndarray:
    """Round float values to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def normal_bf16(shape, std=1.0, seed=0, cid=0, tid=0, layer=0) -> np.ndarray:
    g = rng(seed, cid, tid, layer)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x)


def weight_bf16(N, K, std=0.02, seed=0, cid=0, layer=0, slot=0) -> np.ndarray:
    """Random-init linear weight [N][K], N(0, std^2), as bf16 bits."""
    return normal_bf16((N, K), std, seed, cid, TID_W, layer * 16 + slot)


def uniform_f32(shape, seed, cid, tid, layer=0) -> np.ndarray:
    return rng(seed, cid, tid, layer).random(size=shape, dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------- token trees

def tree_parents(T: int, kind: str, depth_cap: int = 48, seed: int = 0, cid: int = 0,
                 layer: int = 0) -> np.ndarray:
    """Parent array of a T-node tree in topological order; node 0 is the root (-1).

    kind "R": random recursive tree, parent uniform over all earlier nodes.
    kind "CB": a chain of d = min(depth_cap, ceil(3T/4)) nodes under the root, then the
      remaining nodes hang off earlier nodes of depth < depth_cap, chosen uniformly.
    kind "RB": each node draws a child budget b in {1..4}; each new node's parent is
      uniform over earlier nodes of depth < depth_cap that still have budget left.
    kind "chain": a single path 0-1-2-...-(T-1).
    """
    g = rng(seed, cid, TID_TREE, layer)
    par = np.full(T, -1, dtype=np.int32)
    depth = np.zeros(T, dtype=np.int64)
    if T <= 1:
        return par
    if kind == "chain":
        par[1:] = np.arange(T - 1, dtype=np.int32)
        return par
    if kind == "R":
        for i in range(1, T):
            par[i] = g.integers(0, i)
        return par
    if kind == "CB":
        d = min(depth_cap, -(-3 * T // 4), T - 1)
        for i in range(1, d + 1):
            par[i] = i - 1
            depth[i] = i
        for i in range(d + 1, T):
            cand = np.nonzero(depth[:i] < depth_cap)[0]
            p = int(cand[g.integers(0, len(cand))])
            par[i] = p
            depth[i] = depth[p] + 1
        return par
    if kind == "RB":
        budget = np.zeros(T, dtype=np.int64)
        nchild = np.zeros(T, dtype=np.int64)
        budget[0] = g.integers(1, 5)
        for i in range(1, T):
            cand = np.nonzero((depth[:i] < depth_cap) & (nchild[:i] < budget[:i]))[0]
            if len(cand) == 0:
                cand = np.nonzero(depth[:i] < depth_cap)[0]
            p = int(cand[g.integers(0, len(cand))])
            par[i] = p
            depth[i] = depth[p] + 1
            nchild[p] += 1
            budget[i] = g.integers(1, 5)
        return par
    raise ValueError(f"unknown tree kind {kind!r}")


def tree_tokens(parents: np.ndarray, V: int, seed: int = 0, cid: int = 0,
                layer: int = 0) -> np.ndarray:
    """Token ids for the tree nodes, uniform in [0, V), distinct among siblings."""
    g = rng(seed, cid, TID_TOK, layer)
    T = len(parents)
    tok = np.zeros(T, dtype=np.int32)
    seen = {}
    for i in range(T):
        p = int(parents[i])
        used = seen.setdefault(p, set())
        while True:
            t = int(g.integers(0, V))
            if t not in used:
                break
        used.add(t)
        tok[i] = t
    return tok


def chain_path(parents: np.ndarray) -> list:
    """Nodes 0, c1, c2, ... of the main chain: at each node, follow its lowest-index child."""
    T = len(parents)
    path = [0]
    cur = 0
    while True:
        kids = [i for i in range(cur + 1, T) if parents[i] == cur]
        if not kids:
            return path
        cur = kids[0]
        path.append(cur)


def deepest_path(parents: np.ndarray) -> list:
    """Nodes from the root to the deepest node (the lowest-index one among equals)."""
    T = len(parents)
    depth = np.zeros(T, dtype=np.int64)
    for i in range(1, T):
        depth[i] = depth[parents[i]] + 1
    cur = int(np.argmax(depth))
    path = [cur]
    while cur != 0:
        cur = int(parents[cur])
        path.append(cur)
    return path[::-1]


def target_logits(parents, tokens, V, L_star, seed=0, cid=0, layer=0, path=None) -> np.ndarray:
    """Seeded target logits [T][V] fp32 with a planted acceptance of L_star nodes.

    Rows are N(0,1). Along the path c0=0, c1, ... (the main chain of lowest-index children
    unless a path is given), the row of c_m gets tokens[c_{m+1}] raised to (row max + 1)
    for m < L_star; the row of c_{L_star} gets a token that no child of c_{L_star} carries
    raised the same way.
    """
    g = rng(seed, cid, TID_LOGIT, layer)
    T = len(parents)
    lg = g.standard_normal(size=(T, V), dtype=np.float32)
    path = chain_path(parents) if path is None else list(path)
    L_star = min(L_star, len(path) - 1)
    for m in range(L_star):
        row = lg[path[m]]
        row[tokens[path[m + 1]]] = row.max() + np.float32(1)
    stop = path[L_star]
    kid_tokens = {int(tokens[i]) for i in range(T) if parents[i] == stop}
    x = 0
    while x in kid_tokens:
        x += 1
    row = lg[stop]
    row[x] = row.max() + np.float32(1)
    return lg


def gumbel_f32(rows, V, seed=0, cid=0, layer=0) -> np.ndarray:
    """Gumbel(0,1) noise -log(-log u), u uniform on (0,1), drawn in fp64 then rounded to fp32."""
    g = rng(seed, cid, TID_GUMBEL, layer)
    u = g.random(size=(rows, V), dtype=np.float64)
    u = np.clip(u, np.finfo(np.float64).tiny, 1.0 - 2.0 ** -53)
    return (-np.log(-np.log(u))).astype(np.float32)


def norm_gain_bf16(H, seed=0, cid=0, layer=0, which=0, random=False) -> np.ndarray:
    """RMSNorm gain: ones for the configs, or 1 + 0.1 N(0,1) when `random` (used by tests)."""
    if not random:
        return bf16_bits(np.ones(H, dtype=np.float32))
    g = rng(seed, cid, TID_NORM, layer * 4 + which)
    return bf16_bits(1.0 + 0.1 * g.standard_normal(H, dtype=np.float32))


# ---------------------------------------------------------------- GPU-side draws

def torch_normal_bf16(shape, std, seed, cid, tid, layer, device):
    """N(0, std^2) bf16 tensor drawn on `device` with a generator keyed like `rng`."""
    import torch
    key = np.random.SeedSequence([seed, cid, tid, layer]).generate_state(2, dtype=np.uint32)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(key[0]) << 32 | int(key[1]))
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=gen)
    return t.to(torch.bfloat16)
