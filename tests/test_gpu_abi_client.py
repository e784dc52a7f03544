"""The C ABI without Python: tests/abi_client (plain C against include/dcp.h
and the HIP runtime) runs a whole decode step -- local counts, owner-filtered
paged writes on every rank, every rank's stripe attention, the merge -- on
seeded bf16 inputs, and its merged output must match the float64 oracle's
unsharded attention within the parity bar."""

import os
import subprocess

import numpy as np
import pytest

from oracle import attention as OA

import gpu_helpers as H

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "abi_client")
SCALE = 1.0 / np.sqrt(192.0)


@pytest.mark.parametrize("N,I,P,q_len,base", [(4, 1, 16, 2, 0), (8, 64, 64, 1, 1), (3, 1, 32, 4, 1)])
def test_c_client_step_matches_the_oracle(tmp_path, N, I, P, q_len, base):
    if not os.path.exists(CLIENT):
        pytest.fail("tests/abi_client is not built: run __graft_entry__.build()")
    lens = np.array([700, 33, 1500, q_len], dtype=np.int32)
    B, Hh = len(lens), 32
    rng = np.random.default_rng(N * 100 + P + q_len)
    q_bits = OA.to_bf16_bits(rng.standard_normal((B, q_len, Hh, 576)).astype(np.float32))
    kv_bits = [OA.to_bf16_bits((rng.standard_normal((int(S), 576)) * 0.5).astype(np.float32)) for S in lens]
    inp = tmp_path / "in.bin"
    with open(inp, "wb") as f:
        f.write(np.array([B, Hh, N, I, P, q_len, base], dtype=np.int32).tobytes())
        f.write(np.array([SCALE], dtype=np.float32).tobytes())
        f.write(lens.astype(np.int32).tobytes())
        f.write(q_bits.tobytes())
        for kb in kv_bits:
            f.write(kb.tobytes())
    out = tmp_path / "out.bin"
    print(f"abi client: N={N} I={I} P={P} q_len={q_len} base={base}", flush=True)
    r = subprocess.run([CLIENT, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr + r.stdout
    got = np.fromfile(out, dtype=np.float32)
    rows = B * q_len * Hh
    assert got.size == rows * 513
    o = got[:rows * 512].reshape(B, q_len, Hh, 512)
    lse = got[rows * 512:].reshape(B, q_len, Hh)
    for b in range(B):
        ref_o, ref_l = OA.full_attention(OA.bf16_bits_to_float(q_bits[b]), OA.bf16_bits_to_float(kv_bits[b]),
                                         int(lens[b]), SCALE)
        H.assert_o_close(o[b], ref_o, f"C client o, request {b}")
        H.assert_lse_close(lse[b], OA.to_base(ref_l, "2" if base else "e"), f"C client lse, request {b}")
