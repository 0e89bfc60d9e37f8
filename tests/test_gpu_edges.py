"""GPU parity at the edges of the operand formats and of the ABI's domain.

* The fp32 global scale g of R (BiLoCo README, section "Kernel": the product
  takes R's codes, its block scales and an fp32 global scale): y = g P + C
  must hold for every finite g the ABI accepts -- 0, negative, tiny (2^-120)
  and huge (1e30) -- on every schedule and batch height, including a
  split-K matrix-core shape.
* Block scales of both operands at the ends of E4M3: every subnormal byte
  0x01..0x07, the zero byte, and 448 (0x7E), reaching every product kernel.
* One workspace serving calls of different shapes one after the other
  (K-slice counts, r = 0 and r > 0 alternating), each result against the
  oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_weight_gemm_amd import binding as B
from bit_weight_gemm_amd import workloads as wl
from bit_weight_gemm_amd.problem import DeviceProblem
from util import check_y

pytestmark = pytest.mark.gpu


def _ref(d):
    return oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"],
                               d["alpha"])


def _all_schedules(d, p, what):
    y_ref = _ref(d)
    scheds = B.biloco_schedules_for(d["M"], d["N"], d["K"], d["r"])
    assert scheds
    for s in scheds:
        print(f"{what} schedule {s}", flush=True)
        p.y.zero_()
        p.gemm(s)
        torch.cuda.synchronize()
        check_y(p.y_float(), y_ref, f"{what} schedule {s}")


@pytest.mark.parametrize("g", [0.0, -0.01, 2.0 ** -120, 1e30], ids=["0", "-0.01", "2^-120", "1e30"])
@pytest.mark.parametrize("M,K,N,r", [(1, 1024, 520, 96), (2, 1024, 520, 96), (8, 1024, 520, 96),
                                     (32, 1024, 520, 96), (32, 4096, 300, 64), (8, 1024, 520, 0)])
def test_global_scale_values(g, M, K, N, r):
    d = wl.make_inputs(M, K, N, r, seed=40 + M + K, g=g)
    assert d["g"] == np.float32(g)
    _all_schedules(d, DeviceProblem(d), f"g={g} {(M, K, N, r)}")


def _act_with_scale_bytes(M, K, targets, rng):
    """bf16 x [M][K] whose 16-element blocks quantise to the E4M3 scale bytes
    `targets` (cycled): the block's largest |x| is exactly 6 * e4m3(byte) (a
    value with at most 6 significant bits, exact in bf16), the others are
    smaller; byte 0 means an all-zero block."""
    nb = K // 16
    x = np.zeros((M, K), np.float32)
    for m in range(M):
        for b in range(nb):
            t = targets[(m * nb + b) % len(targets)]
            if t == 0:
                continue
            e, mt = t >> 3, t & 7
            v = mt * 2.0 ** -9 if e == 0 else (1 + mt / 8) * 2.0 ** (e - 7)
            blk = rng.uniform(-1, 1, 16) * 6 * v * 0.97
            blk[rng.integers(16)] = 6 * v * (1 if rng.random() < 0.5 else -1)
            x[m, 16 * b:16 * b + 16] = blk
    return wl.to_bf16_bits(x)


R_SCALE_SETS = {
    "r-subnormal": [0x01, 0x02, 0x03, 0x04, 0x05, 0x06, 0x07, 0x00],
    "r-448": [0x7E],
    "r-mixed": [0x00, 0x01, 0x07, 0x08, 0x38, 0x70, 0x7D, 0x7E],
}
ACT_SCALE_SETS = {
    "a-subnormal": [0x01, 0x02, 0x03, 0x04, 0x05, 0x06, 0x07],
    "a-448": [0x7E],
    "a-mixed": [0x00, 0x01, 0x05, 0x07, 0x08, 0x30, 0x50, 0x7E],
}


@pytest.mark.parametrize("rset", list(R_SCALE_SETS))
@pytest.mark.parametrize("aset", list(ACT_SCALE_SETS) + ["a-normal"])
@pytest.mark.parametrize("M", [1, 2, 8, 32])
def test_scale_byte_edges(rset, aset, M):
    K, N = 1024, 264
    rng = np.random.default_rng(M * 31 + len(rset) + len(aset))
    for r in (0, 64):
        d = wl.make_inputs(M, K, N, r, seed=M + r)
        pat = np.array(R_SCALE_SETS[rset], np.uint8)
        d["wscales"] = np.resize(pat, (N, K // 16)).copy()
        if aset != "a-normal":
            d["x"] = _act_with_scale_bytes(M, K, ACT_SCALE_SETS[aset], rng)
            # the quantiser really produces those bytes
            _, sc = oracle.quant_act_fp4(d["x"])
            want = set(ACT_SCALE_SETS[aset])
            assert set(np.unique(sc).tolist()) == want, (sorted(set(np.unique(sc).tolist())), want)
        p = DeviceProblem(d)
        _all_schedules(d, p, f"{rset} {aset} M={M} r={r}")


def test_one_workspace_alternating_shapes():
    """Calls of different shapes on one zero-filled workspace, one after the
    other: z over 5 and over 14 K-slices (an in-launch exchange, then a
    launch of its own), r = 0 with a split K between them, M = 1 schedules
    as well; each call's y against the oracle, twice round."""
    shapes = [(8, 5120, 256, 512), (8, 13824, 256, 512), (32, 13824, 200, 0), (8, 5120, 256, 512),
              (1, 5120, 512, 512), (32, 8192, 300, 1024), (1, 5120, 512, 0), (2, 3072, 300, 40)]
    probs = []
    for i, (M, K, N, r) in enumerate(shapes):
        d = wl.make_inputs(M, K, N, r, seed=600 + i)
        probs.append((d, DeviceProblem(d), _ref(d)))
    need = max(p.ws_bytes for _, p, _ in probs)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    for rnd in range(2):
        for i, (d, p, y_ref) in enumerate(probs):
            for s in B.biloco_schedules_for(d["M"], d["N"], d["K"], d["r"]):
                print(f"round {rnd} shape {shapes[i]} schedule {s}", flush=True)
                p.y.zero_()
                p.gemm(s, ws=ws)
                torch.cuda.synchronize()
                check_y(p.y_float(), y_ref, f"round {rnd} {shapes[i]} schedule {s}")
