"""CPU tests of the C-ABI library's host logic (no GPU calls) and of the inputs."""

import ctypes as C
import math
import os
import re

import numpy as np
import pytest

from oracle import gpt
from oracle.configs import ORACLE_CONFIGS
from persistent_transformer_train_amd import configs, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def ofa():
    from persistent_transformer_train_amd import ofa as mod
    return mod


def header_functions():
    src = open(os.path.join(ROOT, "include", "ofa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ofa_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol(ofa):
    names = header_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(ofa._lib, n), n
    assert set(names) == set(ofa.EXPORTED)


def spec_for(name):
    c = configs.CONFIGS[name]
    o = ORACLE_CONFIGS[name]
    return c, o


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_registry_matches_oracle_table(name):
    c, o = spec_for(name)
    assert c["n_layer"] == o.n_layer and c["d_model"] == o.d_model and c["n_head"] == o.n_head
    assert c["d_ff"] == o.d_ff and c["vocab"] == o.vocab and c["n_pos"] == o.n_pos
    assert bool(c["mlp_gated"]) == o.mlp_gated and bool(c["tied_head"]) == o.tied_head
    assert bool(c["has_bias"]) == o.has_bias and c["batch"] == o.batch and c["seq"] == o.seq
    assert c["lr"] == pytest.approx(o.lr) and c["total_steps"] == o.total_steps
    assert (c["lr_schedule"] == configs.LR_COSINE) == (o.lr_schedule == "cosine")


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_param_layout_matches_oracle(ofa, name):
    cfg = ofa.make_config(configs.CONFIGS[name])
    lib_layout = ofa.layout(cfg)
    or_layout = gpt.param_layout(ORACLE_CONFIGS[name])
    assert len(lib_layout) == len(or_layout)
    off = 0
    for (ln, lo, lnum, lk), (on, oshape, ok) in zip(lib_layout, or_layout):
        assert ln == on and lk == ok and lnum == int(np.prod(oshape)) and lo == off
        off += lnum
    assert ofa.ofa_param_count(C.byref(cfg)) == gpt.n_params(ORACLE_CONFIGS[name])


def test_param_counts():
    # 162,716,160 for the GPT-2 layout at 50,304 tokens (biases, learned positions, untied head);
    # 57,705,472 for the tied RoPE / gated model -- the "57.7M" of the RTX 3090 page's "Run" record
    assert gpt.n_params(ORACLE_CONFIGS["c3"]) == 162_716_160
    assert gpt.n_params(ORACLE_CONFIGS["c2"]) == 57_705_472
    assert round(gpt.n_params(ORACLE_CONFIGS["c2"]) / 1e6, 1) == 57.7
    assert gpt.n_params(ORACLE_CONFIGS["c1"]) == 136_960


def test_validate_rejects_bad_configs(ofa):
    buf = C.create_string_buffer(256)
    bad = [dict(d_model=65), dict(n_head=5), dict(seq=600), dict(precision=7), dict(vocab=250),
           dict(beta1=1.5), dict(exec_mode=9)]
    for kw in bad:
        cfg = ofa.make_config(configs.get("c1", **kw))
        assert ofa.ofa_validate_config(C.byref(cfg), buf, 256) == ofa.OFA_E_ARG, kw
        assert buf.value, kw
        assert ofa.ofa_workspace_bytes(C.byref(cfg)) == 0
    for name in ("c1", "c2", "c3", "c4", "c5"):
        cfg = ofa.make_config(configs.CONFIGS[name])
        assert ofa.ofa_validate_config(C.byref(cfg), buf, 256) == ofa.OFA_OK, buf.value
        assert ofa.ofa_workspace_bytes(C.byref(cfg)) > 4 * ofa.ofa_param_count(C.byref(cfg))


def test_task_budget_is_64_bit(ofa):
    # "A longer run exposed a scheduler overflow" (A100 reproduction page): 4,194,304
    # iterations x 2,225 tasks per token wrapped a 32-bit product at 333,659 tokens
    out = C.c_uint64()
    assert ofa.ofa_task_budget(4_194_304, 2_225, C.byref(out)) == ofa.OFA_OK
    assert out.value == 9_332_326_400
    wrapped = out.value % 2 ** 32
    assert wrapped == 742_391_808
    assert wrapped // 2_225 == 333_659
    assert ofa.ofa_task_budget(2 ** 62, 4, C.byref(out)) == ofa.OFA_E_OVERFLOW


# ---------------------------------------------------------------- synthetic inputs

def test_streams_deterministic_and_in_range():
    for name in ("c1", "c2", "c3"):
        kind, cid = configs.STREAMS[name]
        c = configs.CONFIGS[name]
        s1 = synth.TokenStream(kind, cid, c["vocab"], c["batch"], c["seq"])
        s2 = synth.TokenStream(kind, cid, c["vocab"], c["batch"], c["seq"])
        a, b = s1.batch(3), s2.batch(3)
        assert a.shape == (c["batch"], c["seq"] + 1) and a.dtype == np.int32
        assert np.array_equal(a, b)
        assert not np.array_equal(a, s1.batch(4))
        assert a.min() >= 0 and a.max() < c["vocab"]
        assert synth.sha256(a) == synth.sha256(b)


def test_zipf_stream_statistics():
    s = synth.TokenStream("zipf", 2, 12288, 64, 1024)
    x = s.batch(0).ravel()
    # rank-1 probability of the truncated Zipf(1.1) law
    k = np.arange(1, 12289, dtype=np.float64)
    p1 = 1.0 / (k ** -1.1).sum()
    assert abs((x == 0).mean() - p1) < 0.01


def test_markov2_follows_its_rule():
    s = synth.TokenStream("markov2", 3, 50304, 2, 64)
    x = s.batch(1).astype(np.int64)
    inv = np.argsort(s.perm)
    for t in range(2, 64):
        r = (inv[x[:, t]] - s.ha[x[:, t - 2]] - s.hb[x[:, t - 1]]) % 50304 + 1
        assert np.all((r >= 1) & (r <= 50304))


def test_init_params_layout_kinds(ofa):
    cfg = ofa.make_config(configs.CONFIGS["c1"])
    lay = ofa.layout(cfg)
    p = synth.init_params([(n, k) for _, _, n, k in lay], 1)
    for name, off, n, kind in lay:
        seg = p[off:off + n]
        if kind == "ones":
            assert np.all(seg == 1)
        elif kind == "zeros":
            assert np.all(seg == 0)
        else:
            assert abs(seg.std() - 0.02) < 0.004


def test_sha256_fips_vectors_and_random_buffers(ofa):
    """The library's SHA-256 against the FIPS 180-4 example digests of "abc" and of
    the 448-bit two-block message, the empty string's digest, and Python's hashlib
    on buffers of every length around the 55/56/64-byte padding boundaries."""
    import hashlib
    assert ofa.sha256(b"abc").hex() == "ba7816bf8f01cfea414140de5dae2223b00361a396177a9cb410ff61f20015ad"
    two = b"abcdbcdecdefdefgefghfghighijhijkijkljklmklmnlmnomnopnopq"
    assert ofa.sha256(two).hex() == "248d6a61d20638b8e5c026930c3e6039a33ce45964ff2167f6ecedd419db06c1"
    assert ofa.sha256(b"").hex() == "e3b0c44298fc1c149afbf4c8996fb92427ae41e4649b934ca495991b7852b855"
    rng = np.random.default_rng(5)
    for n in list(range(50, 140)) + [4096, 100003]:
        data = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert ofa.sha256(data) == hashlib.sha256(data).digest(), n


def test_checkpoint_header_and_size(ofa):
    assert C.sizeof(ofa.ofa_checkpoint_header) == 256
    cfg = ofa.make_config(configs.CONFIGS["c1"])
    P = ofa.ofa_param_count(C.byref(cfg))
    assert ofa.ofa_checkpoint_bytes(C.byref(cfg)) == 256 + 12 * P


def _selftest(ofa, cfg, program, workers, n_inst, base, per_die, seed=3, n_cu=256):
    msg = C.create_string_buffer(256)
    rc = ofa.ofa_sched_selftest(C.byref(ofa.make_config(cfg)), program, workers, n_cu, n_inst, base, per_die, seed,
                                msg, 256)
    return rc, msg.value.decode()


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
@pytest.mark.parametrize("per_die", [1, 0], ids=["per_die_release", "per_ticket_release"])
def test_scheduler_protocol_on_cpu_threads(ofa, name, per_die):
    """The persistent scheduler's protocol on host threads with the real phase
    tables of each workload's training step (a 256-CU device): every tile runs
    once, after every tile of its dependencies; counters start just below 2^32
    so a 32-bit counter would wrap inside the run.  For the training program the
    self-test first audits the AdamW ranges: they cover every parameter once, and
    each depends transitively on every phase that writes its gradients or reads
    its weights (a build with one layer range's LayerNorm-parameter dependency
    removed fails it, naming the input-gradient product left unordered)."""
    cfg = configs.CONFIGS[name]
    rc, msg = _selftest(ofa, cfg, 0, 40, 2, 2 ** 32 - 10, per_die)
    assert rc == ofa.OFA_OK, msg
    rc, msg = _selftest(ofa, cfg, 1, 24, 2, 2 ** 32 - 3, per_die)   # the evaluation program
    assert rc == ofa.OFA_OK, msg


@pytest.mark.parametrize("per_die", [1, 0], ids=["per_die_release", "per_ticket_release"])
def test_scheduler_protocol_with_split_products(ofa, per_die):
    """c3 on 256 CUs runs the MLP's second product (192 tiles) as two k-half
    phases whose partial sums the next LayerNorm adds; on a 128-CU device it
    stays one phase (one phase per layer fewer).  Protocol and AdamW audit as
    above, on both programs."""
    cfg = configs.CONFIGS["c3"]
    rc, msg = _selftest(ofa, cfg, 0, 40, 2, 2 ** 32 - 10, per_die, n_cu=256)
    assert rc == ofa.OFA_OK, msg
    rc0, msg0 = _selftest(ofa, cfg, 0, 40, 2, 2 ** 32 - 10, per_die, n_cu=128)
    assert rc0 == ofa.OFA_OK, msg0
    n_split, n_plain = (int(m.split()[1]) for m in (msg, msg0))
    assert n_split == n_plain + cfg["n_layer"], (msg, msg0)


def test_scheduler_selftest_catches_an_early_count(ofa):
    """A release that counts a tile before its work is done must be caught."""
    caught = 0
    for seed in range(4):
        rc, msg = _selftest(ofa, configs.CONFIGS["c1"], 0, 32, 3, 0, 2, seed)
        caught += rc == ofa.OFA_E_STATE and "before every tile finished" in msg
    assert caught >= 1
