"""Writes worked_examples.json: hand-derived decodes of a few keys whose P values and E4M3 roundings
are fixed by the mathematics alone. Uses only the Python standard library (no oracle, no GPU code).

Passages (vLLM API page vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.attn_sparse,
module docstring and SparseDcpDecode.merge): P is 448 times exp2 of the logit minus the running
maximum (log2 units), rounded to E4M3 before it multiplies V; the row sum takes the unrounded P;
o = sum * k_scale / total; LSE = max + log2(total / 448), reported in natural log.

Construction: q is 1.0 at rope column 512 and 0 elsewhere; key j's rope byte 0 holds the E4M3 code
of a_j and its other rope bytes are 0, so with scale = k_scale = 1 the natural-log logit of key j is
exactly a_j. Key j's 512 latent bytes all hold the code of v_j. With one split and one chunk the
running maximum is a* = max a_j, so P_j = 448 * exp(a_j - a*). The E4M3 rounding of each P_j is read
off the E4M3 grid by hand (spacing 32 in [256, 448), 16 in [128, 256), 8 in [64, 128), 0.5 in [4, 8),
2^-9 below 2^-6) and written into each example with its neighbours.
"""
import json
import math
import os

# E4M3 codes (OCP E4M3FN: sign, 4 exponent bits with bias 7, 3 mantissa bits)
CODE = {
    0.0: 0x00,      # zero
    0.40625: 0x2D,  # 1.625 * 2^-2: exponent field 5, mantissa 5
    0.46875: 0x2F,  # 1.875 * 2^-2: exponent field 5, mantissa 7
    0.5: 0x30,      # 1.0 * 2^-1
    1.0: 0x38,      # 1.0 * 2^0
    1.5: 0x3C,      # 1.5 * 2^0
    2.0: 0x40,      # 1.0 * 2^1
    3.0: 0x44,      # 1.5 * 2^1
    -0.5: 0xB0,
    -1.0: 0xB8,
    -4.5: 0xC9,     # -(1.125 * 2^2): exponent field 9, mantissa 1
    -11.0: 0xD3,    # -(1.375 * 2^3): exponent field 10, mantissa 3
}

EXAMPLES = [
    # name, logits a_j, latent values v_j, hand-rounded E4M3 P_j, how the rounding was read
    ("round_down", [0.40625, 0.0], [1.0, -1.0], [448.0, 288.0],
     "P_1 = 448 exp(-0.40625) = 298.43; neighbours 288, 320 -> 288"),
    ("round_up", [0.46875, 0.0], [2.0, -0.5], [448.0, 288.0],
     "P_1 = 448 exp(-0.46875) = 280.35; neighbours 256, 288 -> 288"),
    ("three_keys", [1.5, 1.0, 0.0], [1.0, 3.0, -1.0], [448.0, 256.0, 96.0],
     "P_1 = 448 exp(-0.5) = 271.73; neighbours 256, 288 -> 256. "
     "P_2 = 448 exp(-1.5) = 99.96; neighbours 96, 104 -> 96"),
    ("mid_range", [0.0, -4.5], [1.0, -1.0], [448.0, 5.0],
     "P_1 = 448 exp(-4.5) = 4.977; neighbours 4.5, 5.0 -> 5.0"),
    ("subnormal", [0.0, -11.0], [1.0, -1.0], [448.0, 0.0078125],
     "P_1 = 448 exp(-11) = 0.0074824 = 3.83 * 2^-9; neighbours 3 and 4 * 2^-9 -> 4 * 2^-9"),
]


def main():
    out = {
        "source": "hand-derived from the P anchor, the E4M3 rounding and the merge of the vLLM API "
                  "page vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.attn_sparse "
                  "(module docstring; SparseDcpDecode.merge); construction in "
                  "make_worked_examples.py",
        "scale": 1.0,
        "k_scale": 1.0,
        "examples": [],
    }
    for name, a, v, p_rounded, note in EXAMPLES:
        top = max(a)
        p = [448.0 * math.exp(x - top) for x in a]
        total = sum(p)
        out["examples"].append({
            "name": name,
            "note": note,
            "logits": a,
            "logit_codes": [CODE[x] for x in a],
            "v": v,
            "v_codes": [CODE[x] for x in v],
            "p_unrounded": p,
            "p_e4m3": p_rounded,
            "o_method": sum(pr * vj for pr, vj in zip(p_rounded, v)) / total,
            "o_exact": sum(pj * vj for pj, vj in zip(p, v)) / total,
            "lse": top + math.log(sum(math.exp(x - top) for x in a)),
        })
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_examples.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
