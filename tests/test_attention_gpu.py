"""RoPE, the bfloat16 KV cache and one-token causal attention on the GPU against
the CPU oracle (readings R19, R21).

RoPE: fp32 outputs bit for bit (the library forms the rotary table on the host
with the same fp64 angle and libm cosine and sine that the oracle takes, so both
sides rotate with identical fp32 values). Cache appends: the bfloat16 caches equal
the oracle's bit for bit. Attention: fp32 softmax and sums against the oracle's
fp64, within the bound the fp32 arithmetic allows,
  |out - ref| <= 2^-24 (2 (hd + 1) smag + 2 (192 + S)) vmag,
smag being the largest scaled sum |q k| and vmag the weighted sum |v| the
oracle reports, and S = ceil(t_max / 64), at least the number of chunks the
kernel splits the context into (the combine adds the chunk outputs in turn;
within a chunk a sum takes at most 12 steps, and the constant 192 covers those
and the two exponentials of each weight).
"""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_bitlinear_w1_amd import bitlinear as bl
from ternary_weight_bitlinear_w1_amd import synth

from _cases import assert_equal, assert_rel, note, seed

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
THETA = 5e5
NH, NKV, HD = 20, 5, 128


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("m", [1, 4, 33])
def test_rope(m):
    note(f"rope m={m}")
    q_cols = NH * HD + 2 * NKV * HD
    x = synth.activations(seed(40, m, 1), m, q_cols)
    pos = np.random.default_rng(m).integers(0, 4096, size=m).astype(np.int64)
    pos[0] = 0
    if m > 1:
        pos[1] = 4095
    if m > 4:
        pos[2], pos[3] = -1, 4096  # outside the rotary's positions: angle 0
    want = oracle.rope(oracle.rope(x, pos, NH, HD, THETA, 0), pos, NKV, HD, THETA, NH * HD)
    xg = gpu(x)
    pg = gpu(pos)
    tab = bl.rope_table(THETA, HD, 4096, DEV)
    bl.rope(xg, pg, NH, HD, tab, 0)
    bl.rope(xg, pg, NKV, HD, tab, NH * HD)
    got = host(xg)
    assert_equal(got, want, "rope")
    assert np.array_equal(got[:, NH * HD + 2 * NKV * HD - NKV * HD:], x[:, NH * HD + NKV * HD:]), "values untouched"


def test_kv_append():
    note("kv append")
    n_slots, tmax, m = 3, 64, 6
    r = np.random.default_rng(41)
    kc = oracle.round_bf16(r.normal(size=(n_slots, NKV, tmax, HD)).astype(np.float32))
    vc = oracle.round_bf16(r.normal(size=(n_slots, NKV, tmax, HD)).astype(np.float32))
    qkv = synth.activations(seed(41, m, 2), m, NH * HD + 2 * NKV * HD)
    slot = np.array([0, 2, 1, 2, 5, 0], dtype=np.int64)   # slot 5 is out of range
    pos = np.array([0, 63, 10, 11, 3, 64], dtype=np.int64)  # position 64 is out of range
    kg, vg = gpu(kc), gpu(vc)
    qg = gpu(qkv)
    bl.kv_append(qg[:, NH * HD:NH * HD + NKV * HD], qg[:, NH * HD + NKV * HD:], gpu(slot), gpu(pos), kg, vg)
    k_ref, v_ref = kc.copy(), vc.copy()
    skipped = oracle.kv_append(k_ref, v_ref, qkv[:, NH * HD:NH * HD + NKV * HD], qkv[:, NH * HD + NKV * HD:], slot,
                               pos, NKV, HD)
    assert skipped == 2
    assert_equal(host(kg).view(np.uint16), k_ref, "key cache")
    assert_equal(host(vg).view(np.uint16), v_ref, "value cache")


def _check_attention(q, kc, vc, slot, pos, what, nh=NH, nkv=NKV):
    tmax = kc.shape[2]
    out = host(bl.attention_decode(gpu(q), gpu(kc), gpu(vc), gpu(slot), gpu(pos), nh))
    ref, vmag, smag, _ = oracle.attention(q, kc, vc, slot, pos, nh, nkv, HD)
    S = (tmax + 63) // 64
    factor = 2.0 ** -24 * (2 * (HD + 1) * np.repeat(smag, HD, axis=1) + 2 * (192 + S))
    err = np.abs(out.astype(np.float64) - ref.astype(np.float64))
    bound = factor * vmag
    assert (err <= bound).all(), f"{what}: max err / bound {np.max(err / np.maximum(bound, 1e-300)):.3f}"
    return out, ref


# (positions, t_max, q scale): one position; chunk edges; a sharp softmax; the full 4096 context; more
# than 64 chunks (the combine's second round)
CASES = [([0, 0], 64, 1.0), ([255, 256, 257], 512, 1.0), ([63, 64, 65, 127], 512, 1.0), ([1000, 31], 1024, 8.0),
         ([4095, 2047, 100, 0], 4096, 1.0), ([5000, 8191], 8192, 1.0)]


@pytest.mark.parametrize("positions,tmax,qscale", CASES)
def test_attention(positions, tmax, qscale):
    note(f"attention positions={positions} tmax={tmax}")
    m = len(positions)
    n_slots = m + 1
    r = np.random.default_rng(seed(42, m, tmax) % (2 ** 32))
    kc = oracle.round_bf16(r.normal(size=(n_slots, NKV, tmax, HD)).astype(np.float32))
    vc = oracle.round_bf16(r.normal(size=(n_slots, NKV, tmax, HD)).astype(np.float32))
    q = (qscale * r.normal(size=(m, NH * HD + 2 * NKV * HD))).astype(np.float32)  # rows as the q|k|v output
    slot = np.arange(1, m + 1, dtype=np.int64)
    pos = np.array(positions, dtype=np.int64)
    _check_attention(q, kc, vc, slot, pos, "attention")


def test_attention_shared_slot_and_out_of_range():
    """Two tokens of one sequence (a chunk of its prompt): each sees positions up
    to its own. A token with a bad slot or position gets zeros."""
    note("attention shared slot, out of range")
    r = np.random.default_rng(43)
    tmax = 300
    kc = oracle.round_bf16(r.normal(size=(2, NKV, tmax, HD)).astype(np.float32))
    vc = oracle.round_bf16(r.normal(size=(2, NKV, tmax, HD)).astype(np.float32))
    q = r.normal(size=(4, NH * HD)).astype(np.float32)
    slot = np.array([1, 1, 7, 0], dtype=np.int64)
    pos = np.array([10, 260, 3, 300], dtype=np.int64)
    out, _ = _check_attention(q, kc, vc, slot, pos, "shared slot")
    assert not out[2:].any()


# (q heads, kv heads, positions): groups of 2, 8 and 1 query heads per kv head, at one to three tokens (one
# and two tokens split a kv head's query heads over several workgroups)
GROUPS = [(8, 4, [300]), (8, 4, [5, 511]), (8, 1, [511]), (8, 1, [0, 77, 400]), (4, 4, [200, 3])]


@pytest.mark.parametrize("nh,nkv,positions", GROUPS)
def test_attention_groups(nh, nkv, positions):
    note(f"attention heads {nh}/{nkv} positions={positions}")
    m, tmax = len(positions), 512
    r = np.random.default_rng(seed(44, nh * 10 + nkv, m) % (2 ** 32))
    kc = oracle.round_bf16(r.normal(size=(m, nkv, tmax, HD)).astype(np.float32))
    vc = oracle.round_bf16(r.normal(size=(m, nkv, tmax, HD)).astype(np.float32))
    q = r.normal(size=(m, nh * HD)).astype(np.float32)
    slot = np.arange(m, dtype=np.int64)
    _check_attention(q, kc, vc, slot, np.array(positions, dtype=np.int64), "attention groups", nh, nkv)
