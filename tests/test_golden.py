"""The stored single-token case (tests/golden/single_token_k512_n1024.txt,
written from the oracle by tests/golden/make_golden.py)."""
import hashlib

import numpy as np
import pytest

import inputs
from tests.golden.make_golden import SINGLE_TOKEN, single_token


def stored():
    out = {}
    with open(SINGLE_TOKEN) as fh:
        for ln in fh:
            if ln.startswith("#"):
                continue
            k, _, v = ln.partition(":")
            out[k.strip()] = v.strip()
    return out


def test_oracle_reproduces_stored_single_token(ora):
    assert single_token() == stored()


@pytest.mark.gpu
def test_gpu_meets_stored_single_token(ora):
    import torch
    import block_scaled_fp8_r9k_amd as r9k
    from tests.gpu_util import assert_close, dev, host
    s = stored()
    a = inputs.activations(0, 1, 512, outliers=False)
    w = inputs.weights(0, 1024, 512)
    wq, ws = r9k.quant_weight(dev(w))
    assert hashlib.sha256(host(wq).tobytes()).hexdigest() == s["w_codes_sha256"]
    assert " ".join("%08x" % v for v in host(ws).view(np.uint32).ravel()) == s["w_scales"]
    aq, as_ = r9k.quant_act(dev(a))
    assert " ".join("%02x" % v for v in host(aq).ravel()) == s["act_codes"]
    assert " ".join("%08x" % v for v in host(as_).view(np.uint32).ravel()) == s["act_scales"]
    c_ref = np.array([int(x, 16) for x in s["c"].split()], np.uint16).reshape(1, 1024)
    c = host(r9k.gemm_fp8_block_qa(dev(a), wq, ws))
    assert_close(ora, c, ora.bf16_value(c_ref).astype(np.float64), "single token vs stored oracle result")
    torch.cuda.synchronize()
