"""Host doorbell to wake-up ("Coppelius training on the RTX 3090", "Host doorbell
to wake-up"): a decode whose every token waits for the host to ring produces the
tokens of an ordinary decode of the same prompt, and the host's ring-to-token
time exceeds the device's wake-to-token time by the round trip of the doorbell
and the progress word."""

import numpy as np
import pytest

from gpu_common import cfg_of, init_of, log, stream_of

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("name,n_new", [("c1", 24), ("m3", 24), ("c4", 32)])
def test_doorbell_decode_matches_and_measures(name, n_new):
    from persistent_transformer_train_amd import ofa
    cfg = cfg_of(name, exec_mode=0)
    prompt = torch.from_numpy(stream_of(name, cfg).prompt(cfg["prompt_len"])).cuda()
    h = ofa.Handle(cfg, init_of(name, cfg))
    ref = torch.zeros(n_new, dtype=torch.int32, device="cuda")
    h.decode(prompt, n_new, ref)
    h.sync()
    got = torch.zeros(n_new, dtype=torch.int32, device="cuda")
    host_us, dev_us = h.decode_doorbell(prompt, n_new, got)
    h.sync()
    h.close()
    assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy())
    host_us, dev_us = np.array(host_us), np.array(dev_us)
    assert np.all(np.isfinite(host_us)) and np.all(dev_us > 0)
    assert np.all(host_us > dev_us)
    trip = host_us - dev_us
    log(f"{name}: ring->token median {np.median(host_us):.1f} us (max {host_us.max():.1f}); device wake->token "
        f"median {np.median(dev_us):.1f} us; doorbell + progress round trip median {np.median(trip):.1f} us "
        f"(max {trip.max():.1f})")


def test_doorbell_needs_persistent_executor():
    from persistent_transformer_train_amd import ofa
    cfg = cfg_of("c1", exec_mode=1)
    h = ofa.Handle(cfg, init_of("c1", cfg))
    prompt = torch.from_numpy(stream_of("c1", cfg).prompt(cfg["prompt_len"])).cuda()
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(ofa.OfaError) as e:
        h.decode_doorbell(prompt, 4, out)
    assert e.value.code == ofa.OFA_E_STATE
    h.close()
