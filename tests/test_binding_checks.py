"""The Python binding refuses buffers that the C ABI would read or write out of
bounds, or misread, before anything reaches the library: a wrong dtype, a
non-contiguous view, a buffer shorter than the tensor list implies, a host
tensor, and weight or presence lists of the wrong length.  Every refusal but
the device one is checked first, so each is exercised here on host tensors."""
import pytest
import torch

import diloco_outer_step_amd as dlc

K, STRIDE = 3, 256
TENSORS = [(0, 0, 100), (128, 128, 70)]  # ends: 198 in theta_global, 198 in a row


def good():
    return dict(
        theta_g=torch.zeros(STRIDE), momentum=torch.zeros(STRIDE), theta_L=torch.zeros((K, STRIDE)),
        codes=torch.zeros((K, STRIDE), dtype=torch.uint8),
        codebook=torch.zeros((K, len(TENSORS), dlc.DLC_N_BUCKETS)),
        range=torch.zeros((K, len(TENSORS), dlc.DLC_RANGE_FIELDS)),
        workspace=torch.zeros(4096, dtype=torch.uint8), sq_norms=torch.zeros((K, len(TENSORS)), dtype=torch.float64),
        accum=torch.zeros((K, STRIDE)))


def call(name, b, weights=(1.0, 1.0, 1.0), present=None):
    if name == "quantize":
        dlc.dlc_quantize(b["theta_g"], b["theta_L"], TENSORS, b["codes"], b["codebook"], b["range"], b["workspace"],
                         present=present)
    elif name == "quantize_range":
        dlc.dlc_quantize_range(b["theta_g"], b["theta_L"], TENSORS, b["range"], b["workspace"], present=present)
    elif name == "quantize_encode":
        dlc.dlc_quantize_encode(b["theta_g"], b["theta_L"], TENSORS, b["range"], b["codes"], b["codebook"],
                                b["workspace"], present=present)
    elif name == "merge":
        dlc.dlc_merge_outer_step(b["theta_g"], b["momentum"], b["codes"], b["codebook"], list(weights), TENSORS)
    elif name == "rda":
        dlc.dlc_rda_outer_step(b["theta_g"], b["momentum"], b["theta_L"], TENSORS, list(weights), b["codes"],
                               b["codebook"], b["range"], b["sq_norms"], b["workspace"])
    elif name == "ring":
        dlc.dlc_ring_outer_step(b["theta_g"], b["momentum"], b["theta_L"], TENSORS, b["accum"], b["codes"],
                                b["codebook"], b["range"], b["workspace"])
    elif name == "broadcast":
        dlc.dlc_broadcast(b["theta_g"], b["theta_L"], TENSORS)
    elif name == "cycle":
        dlc.dlc_outer_cycle(b["theta_g"], b["momentum"], b["theta_L"], TENSORS, [0, 2], [list(weights)], b["codes"],
                            b["codebook"], b["range"], b["workspace"])
    else:
        raise KeyError(name)


CALLS = ["quantize", "quantize_range", "quantize_encode", "merge", "rda", "ring", "broadcast", "cycle"]
USES = {
    "quantize": {"theta_g", "theta_L", "codes", "codebook", "range", "workspace"},
    "quantize_range": {"theta_g", "theta_L", "range", "workspace"},
    "quantize_encode": {"theta_g", "theta_L", "codes", "codebook", "range", "workspace"},
    "merge": {"theta_g", "momentum", "codes", "codebook"},
    "rda": {"theta_g", "momentum", "theta_L", "codes", "codebook", "range", "sq_norms", "workspace"},
    "ring": {"theta_g", "momentum", "theta_L", "accum", "codes", "codebook", "range", "workspace"},
    "broadcast": {"theta_g", "theta_L"},
    "cycle": {"theta_g", "momentum", "theta_L", "codes", "codebook", "range", "workspace"},
}


def mutations(name):
    """(buffer, replacement, message fragment) for every buffer the call uses."""
    out = []
    for buf in sorted(USES[name]):
        t = good()[buf]
        other = torch.float64 if t.dtype != torch.float64 else torch.float32
        out.append((buf, t.to(other), "must be"))
        if t.dim() == 2:
            out.append((buf, t.t().contiguous().t(), "contiguous" if t.shape[0] != t.shape[1] else "must"))
        if buf == "workspace":
            continue  # its size is the library's check (DLC_ERR_WORKSPACE)
        # too short for the tensor list: half the row length, or half the elements
        short = t[:, : t.shape[1] // 2].contiguous() if t.dim() == 2 else t.flatten()[: t.numel() // 2].clone()
        out.append((buf, short, ""))
    return out


@pytest.mark.parametrize("name", CALLS)
def test_host_tensors_are_refused(name):
    with pytest.raises(ValueError, match="device tensor"):
        call(name, good())


@pytest.mark.parametrize("name", CALLS)
def test_wrong_dtype_layout_or_size_is_refused_before_the_device_check(name):
    for buf, bad, msg in mutations(name):
        b = good()
        b[buf] = bad
        with pytest.raises((ValueError, TypeError)) as e:
            call(name, b)
        assert "device tensor" not in str(e.value), (name, buf, str(e.value))
        if msg:
            assert msg in str(e.value), (name, buf, str(e.value))


@pytest.mark.parametrize("name", ["merge", "rda", "cycle"])
@pytest.mark.parametrize("weights", [(1.0, 1.0), (1.0, 1.0, 1.0, 1.0)])
def test_weight_lists_must_hold_one_value_per_learner(name, weights):
    with pytest.raises(ValueError, match=f"holds {len(weights)} values for {K} learners"):
        call(name, good(), weights)


@pytest.mark.parametrize("name", ["quantize", "quantize_range", "quantize_encode"])
def test_presence_lists_must_hold_one_value_per_learner(name):
    with pytest.raises(ValueError, match="present holds 2 values"):
        call(name, good(), present=[1, 1])


def test_merge_weights_lists_must_match():
    with pytest.raises(ValueError, match="arrival holds"):
        dlc.dlc_merge_weights([1.0, 2.0], [0.0], 1, 0.0)


def test_a_codes_buffer_of_another_shape_is_refused():
    b = good()
    b["codes"] = torch.zeros((K, STRIDE + 64), dtype=torch.uint8)
    with pytest.raises(ValueError, match="shape"):
        call("quantize", b)
