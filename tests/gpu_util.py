"""Helpers shared by the GPU parity tests: device upload, layout marshalling, metrics."""
import numpy as np
import torch

DEV = torch.device("cuda:0")


def bf16_dev(bits) -> torch.Tensor:
    a = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)


def bits_np(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(DEV)


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32))).to(DEV)


def u8_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.uint8))).to(DEV)


def upload_weights(W: dict) -> dict:
    return {k: bf16_dev(v) for k, v in W.items()}


def upload_cache(Kp, Vp, Pcap=None):
    """Logical [Hkv, P, hd] K and V -> device Kp [Hkv, Pcap, hd] and Vt [Hkv, hd, Pcap]."""
    Hkv, P, hd = Kp.shape
    Pcap = P if Pcap is None else Pcap
    assert Pcap % 8 == 0 and Pcap >= P
    K = np.zeros((Hkv, Pcap, hd), np.uint16)
    Vt = np.zeros((Hkv, hd, Pcap), np.uint16)
    K[:, :P] = Kp
    Vt[:, :, :P] = Vp.transpose(0, 2, 1)
    return bf16_dev(K), bf16_dev(Vt)


def cache_logical(Kd: torch.Tensor, Vtd: torch.Tensor):
    """Device cache -> logical [Hkv, Pcap, hd] K and V bit arrays."""
    return bits_np(Kd), np.ascontiguousarray(bits_np(Vtd).transpose(0, 2, 1))


def maxrel(got, ref) -> float:
    """max |got - ref| / max |ref| over a whole tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def maxrel_rows(got, ref) -> float:
    """The largest per-row relative error: max over rows of max|got_row - ref_row| /
    max|ref_row| (the last axis is the row). A row whose reference is all zeros is
    measured in absolute terms. Never below maxrel of the whole tensor: the row holding
    the largest difference has a reference maximum no larger than the tensor's."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    got = got.reshape(-1, got.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    den = np.max(np.abs(ref), axis=1)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.max(np.abs(got - ref), axis=1) / den))


def sample_excused(p_row, ref_token: int, margin: float) -> bool:
    """Whether a sampled token that differs from the oracle's draw is excused: the
    oracle's u times the total lies within the device's rounding of a cumulative
    boundary. The device sums float32 tile masses (relative error far below 2e-5) and,
    inside the 256-id tile of the crossing, the bf16-stored probabilities (each within
    2^-9 relative), so a boundary may move by up to 2^-9 of that tile's mass; the band is
    twice that, taken over the tiles of the token and of the id before it."""
    p_row = np.asarray(p_row, np.float64)
    t = {ref_token // 256, max(ref_token - 1, 0) // 256}
    mass = max(float(p_row[256 * j:256 * j + 256].sum()) for j in t)
    return margin <= 2.0 ** -8 * mass + 2e-5 * float(p_row.sum())


def near_tie(u_row: np.ndarray) -> bool:
    """Top-2 gap of the oracle's tempered logits within 1e-3 max(1, |u_top|)."""
    top2 = np.partition(u_row, -2)[-2:]
    return (top2[1] - top2[0]) <= 1e-3 * max(1.0, abs(top2[1]))


def argmax_mismatch_unexcused(am_gpu, am_ref, u) -> int:
    bad = 0
    for i in np.nonzero(np.asarray(am_gpu) != np.asarray(am_ref))[0]:
        if not near_tie(u[i]):
            bad += 1
    return bad


_workloads = {}


def workload(name):
    """(cfg, W bits, W with E converted to float64 for the oracle, device weights) of one
    named full-size workload; one at a time is kept (each holds a 1 GiB vocabulary table),
    shared by the test modules that run in a row."""
    import dg_inputs as di
    import oracle as O

    if name not in _workloads:
        _workloads.clear()
        cfg = di.config(name)
        W = di.weights(cfg)
        W64 = dict(W)
        W64["E"] = O.from_bf16(W["E"])
        _workloads[name] = (cfg, W, W64, upload_weights(W))
    return _workloads[name]
