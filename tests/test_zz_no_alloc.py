"""ckv_decode_step_static -- the decode step whose workspace is the
library's own device array (for callers that cannot allocate) -- against
ckv_decode_step with a caller workspace: two calls in a row on one GPU, the
second with a smaller batch, each compared bit for bit (same kernels, same
inputs: outputs, top-k lists, every cache byte and the status words)."""
import numpy as np
import pytest

from harness import dev, device_layer
from workloads import get_config, make_decode_inputs, make_layer_weights

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_kv_sparse_amd  # noqa: F401


def _bytes(t):
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.view(torch.int16)
    return t.numpy().copy()


@pytest.mark.parametrize("name", ["c5", "c5_c128a", "c5_two_lane"])
def test_static_workspace_step_equals_workspace_step(name):
    from compressed_kv_sparse_amd import _lib as L
    cfg = get_config(name).with_(batch=8, comp_cap=512 if name == "c5_c128a" else 8192, seed=101,
                                 name=f"static_{name}")
    r = cfg.ratio
    n = np.array([32768, 20001, 4100, 131, 9, 30000, 12345, 65536][:cfg.batch], np.int64)
    n = np.minimum(n, cfg.comp_cap * r)
    inp = make_decode_inputs(cfg, n_ctx=n)
    wts = make_layer_weights(cfg)
    stream = torch.cuda.current_stream().cuda_stream
    for B in (8, 5):   # two calls in a row, the second smaller
        ref = device_layer(cfg, wts, inp.cache)
        got = device_layer(cfg, wts, inp.cache)
        x, u, q, pos = dev(inp.x[:B]), dev(inp.u[:B]), dev(inp.q[:B]), dev(inp.pos[:B])
        qI = dev(inp.qI[:B]) if r == 4 else None
        w = dev(inp.w[:B]) if r == 4 else None
        out_r, tk_r = ref.decode_step(x, u, q, qI, w, pos, B=B)
        out_g = got.new_out(B)
        tk_g = torch.full((B, cfg.top_k), -7, dtype=torch.int32, device="cuda") if r == 4 else None
        rc = L.decode_step_static(got.desc, got.weights, got.cache, x, u, q, qI, w, pos, B, tk_g, out_g, stream)
        assert rc == 0, L.strerror(rc)
        torch.cuda.synchronize()
        print(f"[static] {name} B={B} done", flush=True)
        np.testing.assert_array_equal(_bytes(out_g), _bytes(out_r))
        if r == 4:
            np.testing.assert_array_equal(_bytes(tk_g), _bytes(tk_r))
        for k in ("raw", "comp", "idx", "st_kv", "st_sc", "ist_kv", "ist_sc", "status", "n_tokens"):
            a, b = getattr(ref, k), getattr(got, k)
            if a is not None:
                np.testing.assert_array_equal(_bytes(b), _bytes(a), err_msg=k)
        assert int(got.status.abs().sum()) == 0
