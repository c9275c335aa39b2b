"""GPU: sequences far longer than the pages' block size (T up to 65536).

The longest context on the pages is GPT-2's 1024 tokens.  These cases run the
kernels' long loops (up to 1024 key tiles per query tile and 1024 query
tiles per key tile, the lazy rescale over many tiles, float32 sums over
65536 keys), where the whole-problem oracle no longer fits in a test; the
oracle's single-row functions (oracle.rows, pinned against the whole-problem
oracle) check what is cheap to compute exactly:
  * o and lse of query rows at the start, the middle and the end;
  * dq of the same rows (a row's dq needs only that row);
  * dk and dv of a block of keys: from the middle for T = 8192, the last
    tile's keys for the longer lengths (a key's gradients need every row
    after it), and at T = 32768 and 65536 also keys 0 .. 127, whose dK/dV
    workgroup walks every query tile of the sequence (the longest loop), from
    the row-blocked oracle (every row's o and lse in float64, then the key
    block's gradients from all rows);
all to the bf16 bar 2e-2 + 2^-8 |ref| (float32: 1e-4) on unit-variance
inputs.  Two identities that hold at any size because each softmax row sums
to one are checked on the whole output as a coarse sanity bound: the keys' dv
sum to the queries' dO and the keys' dk sum to zero, per (b, h) and column,
to within 2^-6 of the summed terms' absolute mass.  (They cannot see a lost
tile at these lengths: a tile's weights are of order 1/T; the key blocks at
both ends of the sequence are the checks for that.)
"""
import numpy as np
import pytest

from gpu_util import default_scale, inputs, to_dev

pytestmark = pytest.mark.gpu

BF16_TOL, BF16_REL, F32_TOL = 2e-2, 2.0 ** -8, 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_self_attention_sdpa_amd as ga
    ga.load_library()


def _close(got, ref, tol, rel, what):
    err = np.abs(got - ref)
    bad = np.argwhere(~(err <= tol + rel * np.abs(ref)))
    assert bad.size == 0, (f"{what}: {len(bad)} elements out of tolerance, first {tuple(bad[0])}: "
                           f"got {got[tuple(bad[0])]}, ref {ref[tuple(bad[0])]}")


@pytest.mark.parametrize("dtype,T,kblock,start", [("bf16", 8192, (4096, 4160), False),
                                                  ("bf16", 32768, None, True),
                                                  ("bf16", 65536, None, True),
                                                  ("f32", 8192, None, False)])
def test_long_sequence_rows_columns_and_sum_rules(dtype, T, kblock, start):
    import causal_self_attention_sdpa_amd as ga
    from oracle import rows
    B, H, hs = 1, 2, 64
    s = default_scale(hs)
    print(f"case long sequence {dtype} B={B} H={H} T={T} hs={hs}", flush=True)
    x = inputs(B, H, T, hs, dtype, seed=777, workload=f"long-t{T}")
    t = {n: to_dev(a, dtype) for n, a in x.items()}
    o, lse = ga.attention_forward(t["q"], t["k"], t["v"], s)
    dq, dk, dv = ga.attention_backward(t["q"], t["k"], t["v"], o, t["do"], lse, s)
    import torch
    torch.cuda.synchronize()
    got = {n: a.float().cpu().numpy().astype(np.float64)
           for n, a in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
    tol, rel = (F32_TOL, 0.0) if dtype == "f32" else (BF16_TOL, BF16_REL)
    sample = [0, 1, 63, 64, T // 2 - 1, T // 2, T - 65, T - 2, T - 1]
    tail = (T - 64, T) if kblock is None else kblock
    for h in range(H):
        q, k, v, dO = (x[n][0, h] for n in ("q", "k", "v", "do"))
        ro, rl = rows.forward_rows(q, k, v, s, sample)
        _close(got["o"][0, h, sample], ro, tol, rel, f"o rows h={h}")
        _close(got["lse"][0, h, sample], rl, 1e-3 if dtype != "f32" else F32_TOL, 0.0,
               f"lse rows h={h}")
        _close(got["dq"][0, h, sample], rows.dq_rows(q, k, v, dO, s, sample), tol, rel,
               f"dq rows h={h}")
        rdk, rdv = rows.dkdv_columns(q, k, v, dO, s, *tail)
        _close(got["dk"][0, h, tail[0]:tail[1]], rdk, tol, rel, f"dk keys {tail} h={h}")
        _close(got["dv"][0, h, tail[0]:tail[1]], rdv, tol, rel, f"dv keys {tail} h={h}")
        # Sum rules over the whole slice.
        gdv, gdk = got["dv"][0, h], got["dk"][0, h]
        assert np.all(np.abs(gdv.sum(0) - dO.sum(0))
                      <= 2.0 ** -6 * (np.abs(gdv).sum(0) + np.abs(dO).sum(0))), f"sum dv h={h}"
        assert np.all(np.abs(gdk.sum(0)) <= 2.0 ** -6 * np.abs(gdk).sum(0)), f"sum dk h={h}"
    if start:
        # Keys 0 .. 127 of head 0: the dK/dV workgroup that walks all T/64 query tiles.
        q, k, v, dO = (x[n][0, 0] for n in ("q", "k", "v", "do"))
        print(f"  key block 0..127 of T={T}: row-blocked oracle", flush=True)
        fo, fl = rows.forward_all_rows(q, k, v, s)
        bdk, bdv = rows.dkdv_block(q, k, v, dO, s, 0, 128, fo, fl)
        _close(got["dk"][0, 0, :128], bdk, tol, rel, f"dk keys 0..127 T={T}")
        _close(got["dv"][0, 0, :128], bdv, tol, rel, f"dv keys 0..127 T={T}")
