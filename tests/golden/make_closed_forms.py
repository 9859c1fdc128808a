"""Writes closed_forms.json: hand-derived worked examples of absorbed MLA whose
expected outputs follow from the definitions in closed form (no oracle code is
used; only Python's math module evaluates the closed forms).

The pages print no numeric worked example, so these cases are derived from the
definitions they give: explicit-decompression attention with the
(d_nope + d_rope)^-1/2 scale and rotate-half RoPE (xxmr.cn/news/206254,
"MLA的计算过程" stage 2A and "MLA的实现": RoPE module, forward_training).
Run:  python tests/golden/make_closed_forms.py
"""
import json
import math
import os

cases = []

# Case 1: two cached tokens, latent score only, unit weights.
# d_c = d_n = d_v = d_r = 2, H = 1, scale = 1/sqrt(2+2) = 1/2.
# c0 = (1,0), c1 = (0,1), k_pe = 0, W_UK = W_UV = I, q_nope = (2 ln 3, 0), q_pe = 0.
# scores: s0 = (2 ln 3) * 1/2 = ln 3, s1 = 0 -> p = (3/4, 1/4); out = p0*c0 + p1*c1.
cases.append({
    "name": "latent_two_tokens",
    "derivation": "s0 = ln3, s1 = 0 -> softmax (3/4, 1/4); V = c",
    "dims": {"num_heads": 1, "d_latent": 2, "d_rope": 2, "d_nope": 2, "d_v": 2},
    "w_uk": [[[1.0, 0.0], [0.0, 1.0]]],
    "w_uv": [[[1.0, 0.0], [0.0, 1.0]]],
    "c_kv": [[1.0, 0.0], [0.0, 1.0]],
    "k_pe": [[0.0, 0.0], [0.0, 0.0]],
    "q_nope": [[2.0 * math.log(3.0), 0.0]],
    "q_pe": [[0.0, 0.0]],
    "expected_out": [[0.75, 0.25]],
})

# Case 2: RoPE part only (W_UK = 0).  d_r = 2 -> one frequency, inv_freq = 1.
# keys k_pe = (1,0) at positions 0 and 1 -> rotated (1,0) and (cos1, sin1);
# query q_pe = (2,0) at position 1 -> rotated (2cos1, 2sin1).
# rope scores: q.k0 = 2cos1, q.k1 = 2(cos^2 1 + sin^2 1) = 2; scale 1/2 ->
# s0 = cos1, s1 = 1; p0 = 1/(1+e^(1-cos1)); out = (p0, 1-p0) with W_UV = I.
p0 = 1.0 / (1.0 + math.exp(1.0 - math.cos(1.0)))
cases.append({
    "name": "rope_relative_position",
    "derivation": "s0 = cos(1), s1 = 1 -> p0 = 1/(1+exp(1-cos 1))",
    "dims": {"num_heads": 1, "d_latent": 2, "d_rope": 2, "d_nope": 2, "d_v": 2},
    "w_uk": [[[0.0, 0.0], [0.0, 0.0]]],
    "w_uv": [[[1.0, 0.0], [0.0, 1.0]]],
    "c_kv": [[1.0, 0.0], [0.0, 1.0]],
    "k_pe": [[1.0, 0.0], [1.0, 0.0]],
    "q_nope": [[0.0, 0.0]],
    "q_pe": [[2.0, 0.0]],
    "expected_out": [[p0, 1.0 - p0]],
})

# Case 3: one cached token (L = 1): softmax over one key is 1, so
# out = W_UV c0 whatever the query.  W_UV = [[1,2],[3,4]], c0 = (0.5, -1).
cases.append({
    "name": "single_token",
    "derivation": "L = 1 -> p = 1 -> out = W_UV c0 = (1*0.5 + 2*-1, 3*0.5 + 4*-1)",
    "dims": {"num_heads": 1, "d_latent": 2, "d_rope": 2, "d_nope": 2, "d_v": 2},
    "w_uk": [[[0.3, -0.7], [1.1, 0.2]]],
    "w_uv": [[[1.0, 2.0], [3.0, 4.0]]],
    "c_kv": [[0.5, -1.0]],
    "k_pe": [[0.25, 0.75]],
    "q_nope": [[1.5, -2.0]],
    "q_pe": [[0.4, 0.9]],
    "expected_out": [[-1.5, -2.5]],
})

# RoPE table values at known angles (d_r = 16 -> inv_freq = 10000^(-i/8)):
# column 0 has inv_freq 1, column 4 has 10000^(-1/2) = 1/100.
rope = {
    "d_rope": 16,
    "entries": [
        {"pos": 0, "col": 0, "cos": 1.0, "sin": 0.0},
        {"pos": 1, "col": 0, "cos": math.cos(1.0), "sin": math.sin(1.0)},
        {"pos": 100, "col": 4, "cos": math.cos(1.0), "sin": math.sin(1.0)},
        {"pos": 3, "col": 0, "cos": math.cos(3.0), "sin": math.sin(3.0)},
    ],
}

out = {"source": "closed forms derived from the definitions; see make_closed_forms.py",
       "cases": cases, "rope_table": rope}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "closed_forms.json"), "w") as f:
    json.dump(out, f, indent=1)
