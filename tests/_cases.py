"""Helpers shared by the oracle pins and the GPU parity tests: reading the
hand-worked golden cases and decoding codes with torch (a library decode,
independent of the oracle's own)."""
import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "handworked.json")


def torch_decode(codes) -> np.ndarray:
    """fp64 values of E4M3 codes via torch.float8_e4m3fn."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).double().numpy()


def _fill(rows, spans, K):
    out = np.zeros((rows, K), dtype=np.uint8)
    for r in range(rows):
        for lo, hi, code in spans[r]:
            out[r, lo:hi] = int(code, 16)
    return out


def golden_cases():
    with open(GOLDEN) as f:
        doc = json.load(f)
    cases = []
    for c in doc["cases"]:
        M, N, K = c["M"], c["N"], c["K"]
        A = _fill(M, c["A_fill"], K)
        if isinstance(c["B_fill"], str):
            spans = json.loads(c["B_fill"].split(":", 1)[1])
            B = _fill(N, [spans] * N, K)
        else:
            B = _fill(N, c["B_fill"], K)
        a_s = np.array(c["a_s"], dtype=np.float32)
        b_s = np.array(c["b_s"], dtype=np.float32)
        if "C" in c:
            C = np.array(c["C"], dtype=np.float64)
        else:  # column_block_tail rule
            C = np.where(np.arange(N) < 128, 128.0, 384.0)[None, :].astype(np.float64)
        cases.append(dict(name=c["name"], A=A, B=B, a_s=a_s, b_s=b_s, C=C,
                          C_bits=c.get("C_bits")))
    return cases


def exact_int_reference(d, K):
    """16 * C as exact int64 for integer-mode inputs: sum_g 2^(u+v+4) * (Ai Bi^T)_g.
    Requires u + v >= -4 (the recipe's exponent ranges)."""
    Ai, Bi, u, v = d["Ai"], d["Bi"], d["u"], d["v"]
    M, N = Ai.shape[0], Bi.shape[0]
    G = (K + 127) // 128
    nb = np.arange(N) // 128
    out = np.zeros((M, N), dtype=np.int64)
    for g in range(G):
        S = Ai[:, 128 * g:128 * g + 128] @ Bi[:, 128 * g:128 * g + 128].T     # int64, exact
        e = u[:, g][:, None] + v[nb, g][None, :] + 4
        assert e.min() >= 0
        out += S << e
    return out
