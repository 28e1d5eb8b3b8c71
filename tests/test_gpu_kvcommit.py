"""KV commit after acceptance (ss_kv_commit) against the oracle, bit for bit.

The acceptance walk runs on the GPU and its device outputs (path, accept length) feed
the commit directly, as in a captured cycle; the whole caches (committed rows and the
untouched rest) are compared with oracle.kv_commit applied to the oracle's own walk.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import gen
from tests.gpu_util import host, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_quantized_draft_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


@pytest.mark.parametrize("T,C,extra,layers,nkv,hd,mode", [
    (64, 2048, 64, 3, 4, 128, "planted"),    # the 7B workload's tree and context
    (48, 100, 0, 2, 2, 64, "planted"),       # C + T == c_stride
    (64, 0, 5, 1, 1, 128, "all"),            # draft == target along the chain: L = depth
    (17, 33, 3, 2, 2, 64, "none"),           # nothing accepted: only the root
    (256, 512, 0, 1, 8, 128, "planted"),     # the 32B workload's tree size
])
def test_kv_commit_bitexact(T, C, extra, layers, nkv, hd, mode):
    print(f"kv_commit T={T} C={C} layers={layers} nkv={nkv} hd={hd} mode={mode}", flush=True)
    seed = T + C
    kind = "chain" if mode == "all" else "CB"
    par = gen.tree_parents(T, kind, seed=seed) if kind == "chain" else gen.tree_parents(T, "CB", 48, seed=seed)
    tok = gen.tree_tokens(par, 5000, seed=seed)
    if mode == "planted":
        tgt = gen.target_logits(par, tok, 5000, min(27, T - 2), seed=seed).argmax(axis=1).astype(np.int32)
    elif mode == "all":
        tgt = np.zeros(T, np.int32)
        for i in range(1, T):
            tgt[par[i]] = tok[i]
    else:
        tgt = np.full(T, -7, np.int32)   # no draft token matches
    path_o, L_o, _ = oracle.accept(par, tok, tgt)
    rng = np.random.default_rng(seed)
    c_stride = C + T + extra
    kc = [rng.integers(0, 1 << 16, (nkv, c_stride, hd), dtype=np.uint16) for _ in range(layers)]
    vc = [rng.integers(0, 1 << 16, (nkv, c_stride, hd), dtype=np.uint16) for _ in range(layers)]
    kt = [rng.integers(0, 1 << 16, (nkv, T, hd), dtype=np.uint16) for _ in range(layers)]
    vt = [rng.integers(0, 1 << 16, (nkv, T, hd), dtype=np.uint16) for _ in range(layers)]
    dkc, dvc = [_u16(a) for a in kc], [_u16(a) for a in vc]
    dkt, dvt = [_u16(a) for a in kt], [_u16(a) for a in vt]
    path, ln, _ = bq.tree_accept(to_dev(par), to_dev(tok), to_dev(tgt))
    bq.kv_commit(dkc, dvc, dkt, dvt, C, path, ln)
    torch.cuda.synchronize()
    assert int(host(ln)[0]) == L_o
    if mode == "all":
        assert L_o == T - 1
    if mode == "none":
        assert L_o == 0
    for l in range(layers):
        rk, rv = oracle.kv_commit(kc[l], vc[l], kt[l], vt[l], path_o, C)
        assert np.array_equal(host(dkc[l]).view(np.uint16), rk), f"layer {l}: K cache differs"
        assert np.array_equal(host(dvc[l]).view(np.uint16), rv), f"layer {l}: V cache differs"
