"""Pins oracle/rope.py's frequencies and pairings against two independent
library implementations of rotary position embedding (the pages name RoPE
without writing it out, so the oracle follows the standard form; these
routines fix what that standard form is):

  interleaved  GPT-J's embedding in transformers: sinusoids from
               create_sinusoidal_positions (base 10000), applied to
               coordinate pairs (2i, 2i+1) by rotate_every_two.
  half         LLaMA's in transformers: LlamaRotaryEmbedding (any base, the
               default rope type) applied to pairs (i, i + d/2) by
               rotate_half.

Both libraries form the angle pos * theta_i in float32, so positions stay
below 2048, where that angle is within ~2.5e-4 rad of the float64 one; a
wrong frequency exponent, a swapped pairing or a sign slip moves outputs by
order one, far past the 2e-3 bar.
"""

import numpy as np
import pytest

from oracle.rope import inv_freq, rope

torch = pytest.importorskip("torch")
transformers = pytest.importorskip("transformers")

POSITIONS = np.array([0, 1, 2, 7, 100, 511, 1000, 2047])
TOL = 2e-3


def _rows(d, seed):
    return np.random.default_rng(seed).standard_normal((len(POSITIONS), 3, d))  # [pos, heads, d]


@pytest.mark.parametrize("d", [64, 128])
def test_interleaved_matches_gptj(d):
    from transformers.models.gptj import modeling_gptj as G
    x = _rows(d, d)
    table = G.create_sinusoidal_positions(int(POSITIONS.max()) + 1, d)   # [pos, d]: sin | cos
    sincos = table[torch.from_numpy(POSITIONS)][None]                     # [1, s, d]
    sin, cos = torch.split(sincos, d // 2, dim=-1)
    t = torch.from_numpy(x).float()[None]                                 # [1, s, heads, d]
    want = G.apply_rotary_pos_emb(t, sin, cos)[0].double().numpy()
    got = rope(x, POSITIONS[:, None], 10000.0, "interleaved")
    assert np.abs(got - want).max() <= TOL


@pytest.mark.parametrize("d,base", [(64, 10000.0), (128, 10000.0), (128, 500000.0)])
def test_half_matches_llama(d, base):
    from transformers import LlamaConfig
    from transformers.models.llama import modeling_llama as L
    cfg = LlamaConfig(hidden_size=4 * d, num_attention_heads=4, head_dim=d, rope_theta=base)
    emb = L.LlamaRotaryEmbedding(cfg)
    x = _rows(d, d + 1)
    t = torch.from_numpy(x).float().permute(1, 0, 2)[None]                 # [1, heads, s, d]
    pos = torch.from_numpy(POSITIONS)[None]
    cos, sin = emb(t, pos)
    q, _ = L.apply_rotary_pos_emb(t, t, cos, sin)
    want = q[0].permute(1, 0, 2).double().numpy()
    got = rope(x, POSITIONS[:, None], base, "half")
    assert np.abs(got - want).max() <= TOL


@pytest.mark.parametrize("d,base", [(64, 10000.0), (128, 500000.0)])
def test_frequencies_match_llama_default(d, base):
    from transformers import LlamaConfig
    from transformers.models.llama import modeling_llama as L
    cfg = LlamaConfig(hidden_size=4 * d, num_attention_heads=4, head_dim=d, rope_theta=base)
    lib = L.LlamaRotaryEmbedding(cfg).inv_freq.double().numpy()
    assert np.allclose(inv_freq(d, base), lib, rtol=1e-6)


def test_library_pins_catch_planted_mistakes():
    """The comparisons above fail for the plausible mistakes: a frequency
    exponent of -i/d instead of -2i/d, the other pairing, and a rotation by
    -pos (all planted in a copy of the oracle's formula, here on the CPU)."""
    from transformers.models.gptj import modeling_gptj as G
    d = 64
    x = _rows(d, 5)
    table = G.create_sinusoidal_positions(int(POSITIONS.max()) + 1, d)
    sin, cos = torch.split(table[torch.from_numpy(POSITIONS)][None], d // 2, dim=-1)
    want = G.apply_rotary_pos_emb(torch.from_numpy(x).float()[None], sin, cos)[0].double().numpy()

    def planted(theta, pairing, sign):
        ang = sign * POSITIONS[:, None, None].astype(np.float64) * theta
        c, s = np.cos(ang), np.sin(ang)
        out = np.empty_like(x)
        if pairing == "interleaved":
            a, b = x[..., 0::2], x[..., 1::2]
            out[..., 0::2], out[..., 1::2] = a * c - b * s, a * s + b * c
        else:
            a, b = x[..., :d // 2], x[..., d // 2:]
            out[..., :d // 2], out[..., d // 2:] = a * c - b * s, a * s + b * c
        return out

    right = inv_freq(d, 10000.0)
    assert np.abs(planted(right, "interleaved", 1) - want).max() <= TOL   # the formula itself
    half_exponent = np.array([10000.0 ** (-i / d) for i in range(d // 2)])
    assert np.abs(planted(half_exponent, "interleaved", 1) - want).max() > 0.5
    assert np.abs(planted(right, "half", 1) - want).max() > 0.5
    assert np.abs(planted(right, "interleaved", -1) - want).max() > 0.5
