"""Shared helpers for the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C ABI binding, compare with the fp64 oracle."""
import sys

import numpy as np

import gla_inputs as gi
import oracle

TOL = {"fp32": 1e-4, "bf16": 2e-2}
# The final state is fp32 for either input dtype and is formed from products
# carried to fp32 accuracy, so it is held to the fp32 rule.
TOL_HT = 1e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(d, dtype):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    out = {}
    for name in ("q", "k", "v"):
        out[name] = torch.from_numpy(d[name]).to(tdt).to(dev).contiguous()
    out["g"] = torch.from_numpy(d["g"]).to(dev).contiguous()
    out["h0"] = None if d["h0"] is None else torch.from_numpy(d["h0"]).to(dev).contiguous()
    out["cu_seqlens"] = None if d["cu_seqlens"] is None else torch.from_numpy(d["cu_seqlens"]).to(dev)
    return out


def run_gpu(d, dtype, scale=None, output_final_state=True, segment_chunks=0, value_tile=0, schedule=0):
    """One forward through the C ABI; asserts that the workspace status word stayed clear."""
    import torch
    import chunkwise_gated_linear_amd as gla
    t = to_device(d, dtype)
    call = gla.GlaCall(t["q"], t["k"], t["v"], t["g"], h0=t["h0"], cu_seqlens=t["cu_seqlens"],
                       scale=scale, output_final_state=output_final_state,
                       segment_chunks=segment_chunks, value_tile=value_tile, schedule=schedule)
    o, ht = call.o, call.ht
    torch.cuda.synchronize()
    assert call.status() == 0, f"status word {call.status():#x} after the call"
    o64 = o.float().cpu().numpy().astype(np.float64)
    ht64 = None if ht is None else ht.cpu().numpy().astype(np.float64)
    return o64, ht64


def run_oracle(d, scale=None, threads=0):
    return oracle.gla_reference(d["q"], d["k"], d["v"], d["g"], h0=d["h0"], cu_seqlens=d["cu_seqlens"],
                                scale=scale, output_final_state=True, threads=threads)


def rms(x):
    return float(np.sqrt(np.mean(np.square(x)))) if x.size else 0.0


def ulp_bf16(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits): 2^(floor(log2|x|) - 7)."""
    m, e = np.frexp(np.abs(x))
    u = np.ldexp(1.0, e - 8)
    return np.where(x == 0, 0.0, u)


def check_close(name, got, ref, tol, out_dtype="fp32", literal=False):
    """The stated rule max|got - ref| <= tol * rms(ref).

    For bf16 outputs each element may additionally differ by half a bf16 ulp,
    the rounding any bf16 result carries (storing the exact result in bf16
    alone can exceed tol * rms on some inputs).  ``literal=True`` also asserts
    the rule without that allowance.
    Returns max|got - ref| / rms(ref).
    """
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    r = rms(ref)
    rel = float(err.max()) / r if r > 0 else float(err.max())
    allow = tol * r
    if out_dtype == "bf16":
        allow = allow + 0.5 * ulp_bf16(np.maximum(np.abs(got), np.abs(ref)))
    bad = err > allow
    assert not np.any(bad), (f"{name}: {int(bad.sum())} elements beyond tol*rms + rounding; "
                             f"max|err| = {rel:.4e} x rms(ref)")
    if literal:
        assert err.max() <= tol * r, f"{name}: max|err| = {rel:.4e} x rms(ref) > {tol}"
    return rel


def rounding_floor(ref):
    """max |bf16(ref) - ref| / rms(ref): the error of the correctly rounded bf16 result."""
    r = rms(ref)
    if r == 0:
        return 0.0
    return float(np.max(np.abs(gi.to_bf16_f32(ref.astype(np.float32)) - ref))) / r
