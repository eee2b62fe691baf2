"""AWQ int4 g32 routed-expert M=1 step parity (E=512, top-k 10, H=2560, I=160)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_mlp_amd as wq
from gpu_common import DEV, dev, f16_dev, gate, host

pytestmark = pytest.mark.gpu
H, I = 2560, 160


@pytest.fixture(scope="module")
def moe():
    d = synth.awq_moe()
    banks = {}
    for ml in (3, 4):
        banks[ml] = tuple(dev(oracle.awq_pack_bank(*d[n], ml)) for n in ("w13", "w2"))
    return d, banks


def run(d, banks, ids, rw=None, ml=3):
    E = d["w13"][0].shape[0]
    rw = d["router_w"] if rw is None else rw
    out, act = wq.moe_awq_m1_run(f16_dev(d["x_bits"]), dev(np.asarray(ids, dtype=np.int32)),
                                 dev(np.asarray(rw, dtype=np.float32)), *banks[ml], E, I, ml)
    return host(out).view(np.uint16), host(act).view(np.uint16)


def f64(bits):
    return oracle.f16_bits_to_f64(bits)


def ulp_dist(a_bits, b_bits):
    a = a_bits.astype(np.int32)
    b = b_bits.astype(np.int32)
    a = np.where(a & 0x8000, 0x8000 - a, a)          # map to a monotone integer line
    b = np.where(b & 0x8000, 0x8000 - b, b)
    return np.abs(a - b)


@pytest.mark.parametrize("ml", [3, 4])
def test_moe_step_parity(moe, ml):
    d, banks = moe
    out, act = run(d, banks, d["ids"], ml=ml)
    ref_out, ref_act = oracle.moe_awq_m1_ref(d["x_bits"], d["ids"], d["router_w"], d["w13"], d["w2"], I)
    gate(f64(act), f64(ref_act), what=f"moe act (W13+SwiGLU) layout {ml}")
    gate(f64(out)[None], f64(ref_out)[None], what=f"moe out layout {ml}")
    # stage-pair: the GPU act through the oracle's W2 stage -> the output differs only by f32-vs-f64 order
    pair_out, _ = oracle.moe_w2_stage_ref(act, d["ids"], d["router_w"], *d["w2"])
    du = ulp_dist(out, pair_out)
    print(f"[parity] moe W2 stage-pair ulp: max {du.max()}, share > 1 ulp {np.mean(du > 1):.2e}")
    assert du.max() <= 4 and np.mean(du > 1) < 1e-2
    da = ulp_dist(act, ref_act)
    print(f"[parity] moe act ulp vs oracle: max {da.max()}, share > 1 ulp {np.mean(da > 1):.2e}")
    assert np.mean(da > 1) < 1e-2


def test_invalid_and_duplicate_ids(moe):
    d, banks = moe
    out, act = run(d, banks, [-1, 512, 100000, -7, 513, 9999, -2, 600, 1 << 20, -100])
    assert np.all(out == 0) and np.all(act == 0)
    ids = np.array(d["ids"])
    ids[3] = -1
    ids[7] = 512
    out, act = run(d, banks, ids)
    assert np.all(act[3] == 0) and np.all(act[7] == 0)
    ref_out, _ = oracle.moe_awq_m1_ref(d["x_bits"], ids, d["router_w"], d["w13"], d["w2"], I)
    gate(f64(out)[None], f64(ref_out)[None], what="moe with invalid ids")
    dup = np.array([ids[0]] * 2 + list(ids[2:]), dtype=np.int32)
    out, act = run(d, banks, dup)
    assert np.array_equal(act[0], act[1])
    ref_out, _ = oracle.moe_awq_m1_ref(d["x_bits"], dup, d["router_w"], d["w13"], d["w2"], I)
    gate(f64(out)[None], f64(ref_out)[None], what="moe with a duplicate id")


def test_single_route_weight_one_equals_y(moe):
    d, banks = moe
    ids = [int(d["ids"][0])] + [-1] * 9
    rw = [1.0] + [0.5] * 9
    out, act = run(d, banks, ids, rw)
    _, y = oracle.moe_w2_stage_ref(act, np.array(ids), np.array(rw, np.float32), *d["w2"])
    assert np.max(ulp_dist(out, y[0])) <= 1


def test_rotating_ids_and_determinism(moe):
    d, banks = moe
    ids_all = synth.awq_rotating_ids(6, 10, 512)
    for ids in ids_all:
        out, act = run(d, banks, ids)
        out2, act2 = run(d, banks, ids)
        assert np.array_equal(out, out2) and np.array_equal(act, act2)
        ref_out, _ = oracle.moe_awq_m1_ref(d["x_bits"], ids, d["router_w"], d["w13"], d["w2"], I)
        gate(f64(out)[None], f64(ref_out)[None], what="moe rotating ids")
