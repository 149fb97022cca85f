"""The entry points captured into a HIP graph and replayed.

Each case runs an entry point once eagerly, captures the same call
(torch.cuda.CUDAGraph, so the call goes to torch's capture stream through
the binding's stream argument) and replays the graph three times.  Before
each replay the program does eager work of its own:
- the output is overwritten with NaN;
- another library call runs on other buffers;
- everything is synchronised.
Every replay must then write exactly what the eager call wrote, bit for bit.
A replay that depended on state left behind by the eager call, by the
previous replay or by the other call would show here, as would a memset node
giving wrong results on later replays.

Only calls that allocate nothing are captured: every SDPA form (the strided
one included), Add & Norm, mha_forward and mha_forward_add_norm with their
workspace given, and mha_forward_noalloc.  With no workspace, mha_forward
allocates stream-ordered memory.
"""

import numpy as np
import pytest

from gpu_util import note, require_gpu, rounded, to_dev, torch
from transformer_head_scaled_amd import libmha, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _dev(rng, shape, dtype, scale=1.0):
    return to_dev(rounded(rng.standard_normal(shape) * scale, dtype)[0], dtype)


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _replay_matches(fn, out, other):
    """fn() writes ``out``; ``other()`` is unrelated eager library work."""
    fn()
    torch.cuda.synchronize()
    ref = out.clone()
    assert torch.isfinite(ref.float()).all(), "eager result not finite"
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(_bits(out), _bits(ref))
        print(f"[graph] replay {r}: {'identical' if same else 'DIFFERS'}", flush=True)
        assert same, f"replay {r} differs from the eager call"
    del g


def _other(rng):
    """An unrelated eager call: unmasked SDPA on its own buffers."""
    Q, K, V = (_dev(rng, (1, 2, 130, 64), "bf16") for _ in range(3))
    O = torch.empty_like(Q)
    return lambda: libmha.sdpa(Q, K, V, out=O)


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_graph_sdpa(mask):
    rng = np.random.default_rng(9100)
    B, h, n, d = 2, 3, 200, 64
    Q, K, V = (_dev(rng, (B, h, n, d), "bf16") for _ in range(3))
    lens = torch.tensor([200, 131], dtype=torch.int32, device="cuda")
    O = torch.empty_like(Q)
    note(f"graph sdpa bf16 {mask} [{B},{h},{n},{d}] lens 200,131")
    _replay_matches(lambda: libmha.sdpa(Q, K, V, mask=mask, seq_lens=lens, out=O), O, _other(rng))


def test_graph_sdpa_strided():
    """mha_sdpa_strided on [B, n, h, d] views of packed projections (the
    layout x·W gives), O written straight into a concat-layout buffer."""
    rng = np.random.default_rng(9107)
    B, n, h, d = 2, 150, 3, 64
    qkv = _dev(rng, (B, n, 3 * h * d), "bf16")
    Q, K, V = (qkv[:, :, j * h * d:(j + 1) * h * d].view(B, n, h, d).transpose(1, 2) for j in range(3))
    concat = torch.empty((B, n, h * d), dtype=torch.bfloat16, device="cuda")
    O = concat.view(B, n, h, d).transpose(1, 2)
    note(f"graph sdpa_strided bf16 causal [{B},{h},{n},{d}] packed QKV, concat out")
    _replay_matches(lambda: libmha.sdpa_strided(Q, K, V, mask="causal", out=O), concat, _other(rng))


def test_graph_sdpa_window():
    rng = np.random.default_rng(9101)
    Q, K, V = (_dev(rng, (2, 2, 300, 64), "bf16") for _ in range(3))
    O = torch.empty_like(Q)
    note("graph sdpa_window bf16 [2,2,300,64] reach 48/16")
    _replay_matches(lambda: libmha.sdpa_window(Q, K, V, 48, 16, out=O), O, _other(rng))


def test_graph_sdpa_f32():
    rng = np.random.default_rng(9102)
    Q, K, V = (torch.from_numpy(rng.standard_normal((1, 2, 70, 64)).astype(np.float32)).cuda()
               for _ in range(3))
    O = torch.empty_like(Q)
    note("graph sdpa f32 [1,2,70,64] causal")
    _replay_matches(lambda: libmha.sdpa(Q, K, V, mask="causal", out=O), O, _other(rng))


def _mha_inputs(rng, B, n_q, n_k, dm, cross):
    x_q = _dev(rng, (B, n_q, dm), "bf16")
    x_kv = _dev(rng, (B, n_k, dm), "bf16") if cross else None
    W = [_dev(rng, (dm, dm), "bf16", dm ** -0.5) for _ in range(4)]
    return x_q, x_kv, W


@pytest.mark.parametrize("case", ["cross", "short"])
def test_graph_forward(case):
    """cross: projection GEMMs, attention, W^O in three launches; short:
    projections and attention in one launch (n <= 64, d_k 64), then W^O."""
    rng = np.random.default_rng(9103)
    if case == "cross":
        B, n_q, n_k, dm, h = 2, 96, 128, 256, 4
    else:
        B, n_q, n_k, dm, h = 4, 40, 40, 256, 4
    x_q, x_kv, W = _mha_inputs(rng, B, n_q, n_k, dm, case == "cross")
    lens = torch.tensor([n_k, 17, n_k, 1][:B], dtype=torch.int32, device="cuda")
    ws = torch.empty(libmha.workspace_size(B, n_q, n_k, dm, h, libmha.MHA_BF16),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((B, n_q, dm), dtype=torch.bfloat16, device="cuda")
    note(f"graph forward {case} B {B} n_q {n_q} n_k {n_k} d_model {dm} h {h}")
    _replay_matches(lambda: libmha.forward(x_q, *W, h, x_kv=x_kv, kv_lens=lens, out=out,
                                           workspace=ws), out, _other(rng))


def test_graph_forward_noalloc():
    rng = np.random.default_rng(9104)
    B, n_q, n_k, dm, h = 2, 96, 128, 256, 4
    x_q, x_kv, W = _mha_inputs(rng, B, n_q, n_k, dm, True)
    out = torch.empty((B, n_q, dm), dtype=torch.bfloat16, device="cuda")
    note(f"graph forward_noalloc B {B} n_q {n_q} n_k {n_k} d_model {dm} h {h}")
    _replay_matches(lambda: libmha.forward_noalloc(x_q, *W, h, x_kv=x_kv, out=out), out,
                    _other(rng))


def test_graph_forward_add_norm():
    rng = np.random.default_rng(9105)
    B, n, dm, h = 2, 80, 256, 4
    x_q, _, W = _mha_inputs(rng, B, n, n, dm, False)
    gamma, beta = _dev(rng, (dm,), "bf16"), _dev(rng, (dm,), "bf16")
    ws = torch.empty(libmha.add_norm_workspace_size(B, n, n, dm, h, libmha.MHA_BF16),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((B, n, dm), dtype=torch.bfloat16, device="cuda")
    note(f"graph forward_add_norm causal B {B} n {n} d_model {dm} h {h}")
    _replay_matches(lambda: libmha.forward_add_norm(x_q, *W, gamma, beta, h, mask="causal",
                                                    out=out, workspace=ws), out, _other(rng))


def test_graph_add_norm():
    rng = np.random.default_rng(9106)
    x, sub = _dev(rng, (300, 1024), "bf16"), _dev(rng, (300, 1024), "bf16")
    gamma, beta = _dev(rng, (1024,), "bf16"), _dev(rng, (1024,), "bf16")
    out = torch.empty_like(x)
    note("graph add_norm bf16 300 x 1024")
    _replay_matches(lambda: libmha.add_norm(x, sub, gamma, beta, out=out), out, _other(rng))
