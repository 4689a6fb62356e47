"""Writes tests/golden/tiny_chain.json: a two-layer residual chain worked by hand.

The case (4 routed experts, top 2, hidden 8, intermediates 4, one group of 4
per row, int4 codes, power-of-two scales) is built so that every value has a
short closed form.  This script only evaluates those closed forms with the
``math`` module; it imports nothing from the oracle or from the library, so the
stored numbers are independent of both.

What is chained (browser demo page "A 3-billion-parameter OCR model. In this
tab.", section "One forward pass, left to right": the decoder's RMSNorm before
each block and the MoE FFN of step 6; the workload definition adds the residual
stream between layers): h_0 = x, z_l = RMSNorm(h_{l-1}) (no gain, eps inside the
square root), h_l = h_{l-1} + MoE_l(z_l).  eps = 5 here so that the first norm
is exactly 3 and a misplaced eps changes every value.

Run from the repository root:  python tests/golden/tiny_chain_closed_forms.py
"""
import json
import math
import os

E, H, I, IS, G = 4, 8, 4, 4, 4
EPS = 5.0
LN2 = math.log(2.0)


def S(v):
    """SiLU(v) = v / (1 + e^-v)."""
    return v / (1.0 + math.exp(-v))


def zeros(*shape):
    if len(shape) == 1:
        return [0] * shape[0]
    return [zeros(*shape[1:]) for _ in range(shape[0])]


def ones(*shape):
    if len(shape) == 1:
        return [1.0] * shape[0]
    return [ones(*shape[1:]) for _ in range(shape[0])]


def sevens(*shape):
    if len(shape) == 1:
        return [7] * shape[0]
    return [sevens(*shape[1:]) for _ in range(shape[0])]


def empty_layer():
    lay = {"router_w": [[0.0] * H for _ in range(E)]}
    for m, (n, k) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        lay[f"{m}_q"] = [zeros(n, k) for _ in range(E)]
        lay[f"{m}_s"] = [ones(n, k // G) for _ in range(E)]
    for m, (n, k) in (("shared_gate", (IS, H)), ("shared_up", (IS, H)), ("shared_down", (H, IS))):
        lay[f"{m}_q"] = zeros(n, k)
        lay[f"{m}_s"] = ones(n, k // G)
    return lay


def fill_unused(lay, experts):
    """Experts the router does not pick hold code 7 everywhere: any leak shows."""
    for e in experts:
        for m, (n, k) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            lay[f"{m}_q"][e] = sevens(n, k)


# ---------------------------------------------------------------- layer 1
L1 = empty_layer()
L1["router_w"][0][0] = 3.0 * LN2          # with z = 2/3: logit ln 4
L1["router_w"][1][0] = 1.5 * LN2          # logit ln 2
L1["gate_q"][0][0][0] = 3; L1["gate_s"][0][0][0] = 0.5      # g = 3 * 2/3 * 1/2 = 1
L1["up_q"][0][0][0] = 3                                      # u = 2
L1["down_q"][0][0][0] = 1                                    # y[0] = h
L1["down_q"][0][1][0] = -1; L1["down_s"][0][1][0] = 0.5      # y[1] = -h/2
L1["gate_q"][1][0][1] = 3                                    # g = 2
L1["up_q"][1][0][2] = 3; L1["up_s"][1][0][0] = 0.5           # u = 1
L1["down_q"][1][2][0] = 2                                    # y[2] = 2h
L1["shared_gate_q"][0][0] = 6; L1["shared_gate_s"][0][0] = 0.25   # g = 6 * 2/3 / 4 = 1
L1["shared_up_q"][0][0] = -3                                      # u = -2
L1["shared_down_q"][3][0] = 1                                     # y[3] = h
fill_unused(L1, (2, 3))

# ---------------------------------------------------------------- layer 2
L2 = empty_layer()
L2["router_w"][2][4] = 1.0                # logit z1[4]
L2["router_w"][3][0] = 1.0                # logit z1[0]
L2["gate_q"][3][0][0] = 1                 # g = z1[0]
L2["up_q"][3][0][4] = 1                   # u = z1[4]
L2["down_q"][3][5][0] = 1                 # y[5] = h
L2["gate_q"][2][0][4] = 1                 # g = z1[4]
L2["up_q"][2][0][1] = 2                   # u = 2 z1[1]
L2["down_q"][2][6][0] = -1; L2["down_s"][2][6][0] = 0.5   # y[6] = -h/2
L2["shared_gate_q"][0][3] = 1             # g = z1[3]
L2["shared_up_q"][0][2] = 1               # u = z1[2]
L2["shared_down_q"][7][0] = 1             # y[7] = h
fill_unused(L2, (0, 1))

X = [2.0] * H

# ---------------------------------------------------------------- closed forms, float64 norm
S1, S2 = S(1.0), S(2.0)
# layer 1: mean(x^2) = 4, sqrt(4 + 5) = 3, z0 = 2/3 everywhere; logits [ln4, ln2, 0, 0]
P1 = [0.5, 0.25, 0.125, 0.125]
# expert 0: h = [2 S1, 0, 0, 0] -> [2 S1, -S1, 0...]; expert 1: h = [S2] -> y[2] = 2 S2;
# shared: h = [-2 S1] -> y[3] = -2 S1
y1 = [0.5 * 2 * S1, 0.5 * -S1, 0.25 * 2 * S2, -2 * S1, 0.0, 0.0, 0.0, 0.0]
h1 = [X[i] + y1[i] for i in range(H)]
r1 = math.sqrt(sum(v * v for v in h1) / H + EPS)
z1 = [v / r1 for v in h1]
# layer 2: logits [0, 0, z1[4], z1[0]]; z1[0] = (2 + S1)/r1 > z1[4] = 2/r1 > 0, so ids [3, 2]
den = 2.0 + math.exp(z1[4]) + math.exp(z1[0])
P2 = [1.0 / den, 1.0 / den, math.exp(z1[4]) / den, math.exp(z1[0]) / den]
y2 = [0.0] * H
y2[5] = P2[3] * S(z1[0]) * z1[4]
y2[6] = P2[2] * -0.5 * S(z1[4]) * 2.0 * z1[1]
y2[7] = S(z1[3]) * z1[2]
h2 = [h1[i] + y2[i] for i in range(H)]

# ---------------------------------------------------------------- bf16-rounded norm, layer 1 only
# 2/3 = 0.101010...b; keeping 8 significant bits rounds up (the dropped bits are 0.1010... > half):
# bf16(2/3) = 171/256.
a = 171.0 / 256.0
e0, e1 = 2.0 ** (3 * a), 2.0 ** (1.5 * a)   # exp of the logits 3 ln2 a and 1.5 ln2 a
dn = e0 + e1 + 2.0
Pb = [e0 / dn, e1 / dn, 1.0 / dn, 1.0 / dn]
y1b = [Pb[0] * 3 * a * S(1.5 * a),            # expert 0: g = 1.5a, u = 3a, down row 0
       Pb[0] * -1.5 * a * S(1.5 * a),         # down row 1, scale 1/2, code -1
       Pb[1] * 2 * 1.5 * a * S(3 * a),        # expert 1: g = 3a, u = 1.5a, down row 2 code 2
       -3 * a * S(1.5 * a),                   # shared: g = 1.5a, u = -3a
       0.0, 0.0, 0.0, 0.0]
h1b = [X[i] + y1b[i] for i in range(H)]

doc = {
    "what": "Hand-worked two-layer residual chain: 4 routed experts, top-2, hidden 8, "
            "intermediates 4, group 4 along K, int4 codes, power-of-two scales, RMSNorm eps 5.",
    "cites": "RMSNorm before each decoder block and the MoE FFN of step 6 (softmax router, greedy "
             "top-k, no renormalisation, SiLU-gated experts, always-on shared expert): browser demo "
             "page 'A 3-billion-parameter OCR model. In this tab.', section 'One forward pass, left to "
             "right'. Codes with one f32 scale per group: same page, 'Four bits, one shared scale'. "
             "The residual add between layers and eps inside the square root are the workload "
             "definition's. The case is ours; the values are the closed forms of "
             "tests/golden/tiny_chain_closed_forms.py, evaluated with the math module only.",
    "derivation": [
        "h0 = 2 everywhere; mean(h0^2) + eps = 9, so z0 = 2/3 everywhere.",
        "Layer 1 logits [3 ln2 * 2/3, 1.5 ln2 * 2/3, 0, 0] = [ln4, ln2, 0, 0], P = [1/2, 1/4, 1/8, 1/8], ids [0, 1].",
        "Expert 0: g = 3*(2/3)*(1/2) = 1, u = 3*(2/3) = 2, h = [2 S(1)]; down rows 0 and 1 give [2 S(1), -S(1)].",
        "Expert 1: g = 3*(2/3) = 2, u = 3*(2/3)*(1/2) = 1, h = [S(2)]; down row 2 gives 2 S(2).",
        "Shared: g = 6*(2/3)/4 = 1, u = -3*(2/3) = -2, h = [-2 S(1)]; down row 3 gives -2 S(1).",
        "y1 = [S(1), -S(1)/2, S(2)/2, -2 S(1), 0, 0, 0, 0]; h1 = h0 + y1.",
        "r1 = sqrt(mean(h1^2) + 5); z1 = h1 / r1. Layer 2 logits [0, 0, z1[4], z1[0]] with z1[0] > z1[4] > 0, so ids [3, 2].",
        "Expert 3: g = z1[0], u = z1[4], down row 5 gives S(z1[0]) z1[4]. Expert 2: g = z1[4], u = 2 z1[1], "
        "down row 6 (code -1, scale 1/2) gives -S(z1[4]) z1[1]. Shared: g = z1[3], u = z1[2], down row 7 gives S(z1[3]) z1[2].",
        "h2 = h1 + [0, 0, 0, 0, 0, P3 S(z1[0]) z1[4], -P2 S(z1[4]) z1[1], S(z1[3]) z1[2]].",
        "bf16 chain (layer 1 only): z0 = bf16(2/3) = 171/256 = a; logits [3 ln2 a, 1.5 ln2 a, 0, 0]; "
        "y1 = [P0 3a S(1.5a), -P0 1.5a S(1.5a), P1 3a S(3a), -3a S(1.5a), 0, 0, 0, 0].",
    ],
    "E": E, "H": H, "I": I, "Is": IS, "group": G, "bits": 4, "eps": EPS, "top_k": 2,
    "x": X,
    "layers": [L1, L2],
    "expected": {
        "z0": [2.0 / 3.0] * H,
        "P1": P1, "ids1": [0, 1], "w1": P1[:2],
        "h1": h1,
        "z1": z1,
        "P2": P2, "ids2": [3, 2], "w2": [P2[3], P2[2]],
        "h2": h2,
        "bf16_one_layer": {"z0": [a] * H, "P1": Pb, "ids1": [0, 1], "w1": Pb[:2], "h1": h1b},
    },
}

if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_chain.json")
    with open(out, "w") as f:   # one top-level key (and one layer tensor) per line
        f.write("{\n")
        items = []
        for k, v in doc.items():
            if k == "layers":
                rows = [",\n".join(f"   {json.dumps(n)}: {json.dumps(t)}" for n, t in lay.items()) for lay in v]
                items.append(f" {json.dumps(k)}: [\n  {{\n" + "\n  },\n  {\n".join(rows) + "\n  }\n ]")
            else:
                items.append(f" {json.dumps(k)}: {json.dumps(v)}")
        f.write(",\n".join(items) + "\n}\n")
    print(out)
