"""The seeded input generators (they hold none of the method's arithmetic):
repeatable per seed and workload, distinct across them."""
import torch

from mixture_experts_layer_07_amd import workloads as wl


def test_device_generators_are_seeded_and_distinct():
    """The large-shape input generators (drawn where the tensors live, here
    on the host) repeat for the same seed and workload, differ across seeds
    and workloads, and round x to the activation dtype."""
    w = wl.Workload("gen", 90, T=37, H=256, E=8, I=128, k=2, method=wl.ROUTE_DEFAULT)
    a = wl.make_x_device(w, 0, "cpu", chunk_rows=16)
    assert a.dtype == torch.bfloat16 and a.shape == (37, 256)
    assert torch.equal(a, wl.make_x_device(w, 0, "cpu", chunk_rows=16))
    assert not torch.equal(a, wl.make_x_device(w, 1, "cpu", chunk_rows=16))
    assert not torch.equal(a, wl.make_x_device(w.with_(cid=91), 0, "cpu", chunk_rows=16))
    assert 0.8 < float(a.float().std()) < 1.2
    lg = wl.make_logits_direct(w)
    assert lg.dtype == torch.float32 and lg.shape == (37, 8)
    assert torch.equal(lg, wl.make_logits_direct(w))
    assert not torch.equal(lg, wl.make_logits_direct(w, 1))
