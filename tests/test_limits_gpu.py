"""mha_sdpa at the supported size limits, checked through closed forms.

The fp64 oracle cannot hold these inputs (one head of 16.7 M keys), so each
case is built so that the exact result has a plain form:

* one key's score exceeds every other by far more than log(n_k): the
  softmax puts (all but 1e-6 of) its weight on that key, so O = V[that key]
  (the one-hot limit of eq. (1), nickwang.xyz §3.2.1);
* Q = 0: every visible score is 0, the weights are uniform and O is the
  mean of the visible value rows (the reduction is done in float64 by
  torch on the device, a library routine);
* one key per head: its weight is exactly 1, so O = V bit for bit.

Limits exercised: one head's K (and V) just under 2 GiB, the largest byte
offsets the kernels form (key split for one query row, the plain path for
100 rows, a key length just below n_k); and B·h at its 2^24 limit.
Inputs are drawn on the device by torch's generator with a fixed seed.
"""

import pytest

from gpu_util import note, require_gpu, torch
from transformer_head_scaled_amd import libmha

pytestmark = pytest.mark.gpu

N_K_MAX = (1 << 24) - 64          # K rows of 64 bf16: 2^31 - 8192 bytes, under the 2 GiB limit
FAR = N_K_MAX - 5                 # the dominant key, near the end


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def big_kv():
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    K = (0.01 * torch.randn(1, 1, N_K_MAX, 64, device="cuda", generator=g)).bfloat16()
    V = torch.randn(1, 1, N_K_MAX, 64, device="cuda", generator=g).bfloat16()
    u = (2.0 * (torch.randint(0, 2, (64,), device="cuda", generator=g) * 2 - 1)).bfloat16()
    K[0, 0, FAR] = u          # score 0.125 · |u|² = 32 against |score| <~ 1 elsewhere
    yield K, V, u
    del K, V
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n_q", [1, 100])
def test_largest_head_one_hot(big_kv, n_q):
    """n_q 1 runs the key split, 100 the two-wave plain path; every row's
    weight sits on key FAR, 16.7 M keys in (offsets near 2^31 bytes)."""
    K, V, u = big_kv
    Q = u.view(1, 1, 1, 64).expand(1, 1, n_q, 64).contiguous()
    note(f"sdpa bf16 one head of {N_K_MAX} keys, n_q {n_q}, one-hot at {FAR}")
    O = libmha.sdpa(Q, K, V, scale=0.125)
    torch.cuda.synchronize()
    exp = V[0, 0, FAR].float()
    err = float((O[0, 0].float() - exp).abs().max())
    print(f"[parity] one-hot at key {FAR} of {N_K_MAX}, n_q {n_q}: max-abs {err:.3e}", flush=True)
    assert err <= 2e-2


@pytest.mark.parametrize("n_q", [1, 100])
def test_largest_head_uniform_with_key_length(big_kv, n_q):
    """Q = 0 and a key length 3 below n_k: O = mean of V over the first
    n_k - 3 rows."""
    K, V, _ = big_kv
    n_eff = N_K_MAX - 3
    Q = torch.zeros(1, 1, n_q, 64, device="cuda", dtype=torch.bfloat16)
    lens = torch.tensor([n_eff], dtype=torch.int32, device="cuda")
    note(f"sdpa bf16 one head of {N_K_MAX} keys, Q = 0, key length {n_eff}, n_q {n_q}")
    O = libmha.sdpa(Q, K, V, scale=0.125, seq_lens=lens)
    torch.cuda.synchronize()
    exp = V[0, 0, :n_eff].double().mean(dim=0)
    err = float((O[0, 0].double() - exp).abs().max())
    print(f"[parity] uniform over {n_eff} keys, n_q {n_q}: max-abs {err:.3e}", flush=True)
    assert err <= 2e-3   # |mean| ~ 3e-4; the bf16 rounding of O is far below this


def test_most_heads_single_key():
    """B·h = 65535 · 256 (just under 2^24) heads of one query and one key,
    d 16: every weight is exactly 1, so O = V bit for bit."""
    B, h = 65535, 256
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    Q, K, V = (torch.randn(B, h, 1, 16, device="cuda", generator=g).bfloat16() for _ in range(3))
    note(f"sdpa bf16 {B}x{h} heads of one key, d 16")
    O = libmha.sdpa(Q, K, V, scale=0.25)
    torch.cuda.synchronize()
    assert torch.equal(O, V)
    del Q, K, V, O
    torch.cuda.empty_cache()
