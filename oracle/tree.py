"""Token tree: structure, ancestor mask and the greedy acceptance walk.

TEST INFRASTRUCTURE ONLY (see the package header).

[Review] §6.3 (SpecInfer): the draft proposes a tree of candidate tokens and one
target pass verifies every root-to-node path; SubSpec makes the tree deep and
narrow (k = 6, depth 48). [Review] §3.2 and [Summary] "Key results" evaluate it with
greedy (temperature 0) decoding.

Readings (the pages do not fix them): node 0 is the root, the last committed
token, whose KV entry is not yet cached; parents[0] = -1 and 0 <= parents[i] < i
(topological order). A node attends to its ancestors and itself. The mask row of
node i is a bitset over tree nodes packed into 64-bit words, least significant bit
first: bit (j mod 64) of word (j div 64) is set iff j is i or an ancestor of i.
"""

import numpy as np


def validate_tree(parents) -> bool:
    p = [int(x) for x in parents]
    if len(p) == 0 or p[0] != -1:
        return False
    return all(0 <= p[i] < i for i in range(1, len(p)))


def tree_depth(parents) -> np.ndarray:
    """depth[0] = 0, depth[i] = depth[parents[i]] + 1."""
    T = len(parents)
    d = np.zeros(T, dtype=np.int32)
    for i in range(1, T):
        d[i] = d[int(parents[i])] + 1
    return d


def tree_mask(parents) -> np.ndarray:
    """Ancestor-or-self bitmask, uint64 [T][ceil(T/64)], built by anc[i] = anc[parent] | {i}."""
    if not validate_tree(parents):
        raise ValueError("parents is not a topologically ordered tree rooted at node 0")
    T = len(parents)
    W = (T + 63) // 64
    anc = [0] * T
    for i in range(T):
        p = int(parents[i])
        anc[i] = (anc[p] if p >= 0 else 0) | (1 << i)
    m = np.zeros((T, W), dtype=np.uint64)
    for i in range(T):
        for w in range(W):
            m[i, w] = (anc[i] >> (64 * w)) & 0xFFFFFFFFFFFFFFFF
    return m


def accept(parents, tokens, target_argmax):
    """Greedy tree acceptance.

    target_argmax[i] is the target's next-token choice after the path ending at node i.
    Starting at the root, repeatedly accept the child (lowest index on ties) whose
    draft token equals the target's choice at the current node; stop when none does.
    Returns (path of accepted nodes excluding the root, accept length L, bonus token),
    where the bonus token is the target's choice at the last accepted node; the
    cycle commits L + 1 tokens.
    """
    T = len(parents)
    path = []
    cur = 0
    while True:
        want = int(target_argmax[cur])
        nxt = -1
        for i in range(cur + 1, T):
            if int(parents[i]) == cur and int(tokens[i]) == want:
                nxt = i
                break
        if nxt < 0:
            break
        path.append(nxt)
        cur = nxt
    return path, len(path), int(target_argmax[cur])


def kv_commit(k_cache, v_cache, k_tree, v_tree, path, C):
    """Commit the accepted tokens' keys and values to the shared cache.

    [Review] §4.1: draft and target share one KV cache; the verification of a cycle
    commits the root and the L accepted nodes (the acceptance walk above). Reading
    (the pages give no procedure): the target's tree K/V rows of the root and of the
    accepted path, which already carry RoPE at positions C + depth, are written in path
    order to cache rows C .. C + L (depth i lands in row C + i); nothing else changes.
    Arrays hold bf16 bits: caches [nkv][c_stride][hd], tree K/V [nkv][T][hd].
    Returns new arrays.
    """
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    for i, node in enumerate([0] + [int(n) for n in path]):
        k[:, C + i, :] = k_tree[:, node, :]
        v[:, C + i, :] = v_tree[:, node, :]
    return k, v
