"""Parity of the Hyper-Connection mixer (ckv_hc_pre / ckv_hc_post, through the
C ABI) with the oracle: the split (pre weights, post gates, Sinkhorn coupling
matrix), the block input and the updated streams, at the Flash shape's hidden
size, on ragged sizes and with saturated mixer rows.  Bars: split values
within 1e-5 relative + 2e-6 absolute (float32 arithmetic against fp64); mixes
within the output format's rounding (bf16: 4e-3 relative) + 1e-5 absolute."""
import numpy as np
import pytest

import oracle as O
from harness import dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SPLIT_TOL = (1e-5, 2e-6)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw(T, D, fmt, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    mix = (rng.standard_normal((T, 24)) * scale).astype(np.float32)
    h = rng.standard_normal((T, 4, D)).astype(np.float32)
    y = rng.standard_normal((T, D)).astype(np.float32)
    if fmt == "bf16":   # bf16-valued draws (low half of the float dropped)
        h = (h.view(np.uint32) & 0xFFFF0000).view(np.float32)
        y = (y.view(np.uint32) & 0xFFFF0000).view(np.float32)
    return mix, h, y


def to_dev(a, fmt):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(torch.bfloat16) if fmt == "bf16" else t


def close(g, r, rtol, atol, what):
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    bad = np.abs(g - r) > atol + rtol * np.abs(r)
    assert not bad.any(), f"{what}: {int(bad.sum())} outside; first {np.argwhere(bad)[:3].tolist()}"


def run_case(T, D, fmt, seed, scale=1.0, sample=None):
    from compressed_kv_sparse_amd import HCMixer
    print(f"[hc] T={T} D={D} {fmt} seed={seed} scale={scale}", flush=True)
    mix, h, y = draw(T, D, fmt, seed, scale)
    m = HCMixer(D, act_fmt=fmt)
    x, coef = m.pre(dev(mix), to_dev(h, fmt))
    hout = m.post(coef, to_dev(h, fmt), to_dev(y, fmt))
    torch.cuda.synchronize()
    xg = x.float().cpu().numpy()
    cg = coef.cpu().numpy()
    hg = hout.float().cpu().numpy()
    rows = range(T) if sample is None else sample
    rt = 4e-3 if fmt == "bf16" else 1e-5
    for t in rows:
        pre, post, comb = O.hc_split(mix[t])
        close(cg[t, :4], pre, *SPLIT_TOL, f"pre t={t}")
        close(cg[t, 4:8], post, *SPLIT_TOL, f"post t={t}")
        close(cg[t, 8:], comb.reshape(-1), *SPLIT_TOL, f"coupling t={t}")
        close(xg[t], O.hc_pre(pre, h[t]), rt, 1e-5, f"x t={t}")
        close(hg[t], O.hc_post(post, comb, h[t], y[t]), rt, 1e-5, f"h_out t={t}")


@pytest.mark.parametrize("T,D,fmt", [(5, 4096, "bf16"), (3, 1000, "bf16"), (7, 64, "f32"), (16, 4096, "f32")])
def test_hc_mixer_matches_the_oracle(T, D, fmt):
    run_case(T, D, fmt, seed=T * 131 + D)


def test_hc_mixer_saturated_rows():
    """Mixer rows of +-30: gates at 0 / 1 and near-permutation coupling."""
    run_case(6, 4096, "bf16", seed=77, scale=30.0)


def test_hc_mixer_prefill_size_sampled():
    """A 4096-token chunk at hidden 4096 (bf16), sampled tokens checked."""
    run_case(4096, 4096, "bf16", seed=4096, sample=[0, 1, 2, 1000, 2047, 2048, 4093, 4095])
