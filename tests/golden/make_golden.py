"""Writes the stored oracle results under tests/golden/ (calls only oracle/
and the seeded input generator).

single_token_k512_n1024.txt: the single-token decode case, one bf16 row of 512
activations ~ N(0,1) (no outliers) against 1024 x 512 weights of
fp32(0.02 N(0,1)) rounded to bf16, seed 0; the oracle's weight block quant,
activation group quant and block GEMM.  Lines: `act_scales` (4 fp32 bit
patterns), `act_codes` (512 codes), `w_scales` (8 x 4 fp32 bit patterns),
`c` (1024 bf16 bit patterns), all hex; `w_codes_sha256` (the 524288 weight
codes are too many to store as text).

Run from the repository root: python -m tests.golden.make_golden
"""
import hashlib
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import inputs  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
SINGLE_TOKEN = os.path.join(HERE, "single_token_k512_n1024.txt")


def single_token():
    a = inputs.activations(0, 1, 512, outliers=False)
    w = inputs.weights(0, 1024, 512)
    wq, ws = oracle.quant_weight(w)
    aq, as_ = oracle.quant_act(a)
    c = oracle.gemm_block(aq, as_, wq, ws)
    return dict(
        act_scales=" ".join("%08x" % v for v in as_.view(np.uint32).ravel()),
        act_codes=" ".join("%02x" % v for v in aq.ravel()),
        w_scales=" ".join("%08x" % v for v in ws.view(np.uint32).ravel()),
        w_codes_sha256=hashlib.sha256(np.ascontiguousarray(wq).tobytes()).hexdigest(),
        c=" ".join("%04x" % v for v in c.ravel()),
    )


def main():
    oracle.build(force=False)
    fields = single_token()
    with open(SINGLE_TOKEN, "w") as fh:
        fh.write("# written by tests/golden/make_golden.py from the oracle; see its docstring\n")
        for k, v in fields.items():
            fh.write(f"{k}: {v}\n")


if __name__ == "__main__":
    main()
