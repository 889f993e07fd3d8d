"""The no-allocation entry point, through the C ABI: spec_verify_noalloc
(workspace in the library's fixed device scratch array) equals spec_verify on
a context (workspace allocated at init) bit for bit, on two calls in a row,
the second with a smaller input, and rejects a shape whose workspace exceeds
the array before launching anything."""
import numpy as np
import pytest
import torch

import device_draft_verification_amd as sv
import specgen
from gpu_helpers import run_gpu, to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


def _noalloc(t, seed, offset):
    zp = t["logits_target"]
    B, G1, _ = zp.shape
    alen = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    toks = torch.full((B, G1), -7, dtype=torch.int32, device="cuda")
    rc = sv.spec_verify_noalloc(t["logits_draft"], zp, t["draft_tokens"], t["temperature"], seed,
                                offset, alen, toks)
    assert rc == sv.binding.SPEC_OK
    torch.cuda.synchronize()
    return dict(accept_len=alen.cpu().numpy(), tokens=toks.cpu().numpy())


@pytest.mark.parametrize("first,second", [
    ((4, {}), (2, dict(batch=8, vocab=32000))),                 # fused draw, then tile draw
    ((5, dict(batch=160, vocab=50000)), (4, dict(batch=130, vocab=20011))),  # vector, then element path
])
def test_noalloc_equals_spec_verify_on_two_calls(first, second):
    for n, (cfg, over) in enumerate((first, second)):
        rec = specgen.config(cfg).replace(**over)
        t = to_device(specgen.generate(rec))
        for seed, offset in ((0, 0), (7, 3)):
            got = _noalloc(t, seed, offset)
            ref = run_gpu(t, seed=seed, offset=offset, with_lse=False)
            assert np.array_equal(got["accept_len"], ref["accept_len"]), (n, rec.name)
            assert np.array_equal(got["tokens"], ref["tokens"]), (n, rec.name)
            assert (got["accept_len"] >= 0).all()
        print(f"\n[noalloc] call {n}: {rec.name} {over} equal to spec_verify", flush=True)
        del t
        torch.cuda.empty_cache()


def test_noalloc_rejects_a_workspace_beyond_the_array():
    # B = 127 keeps the two-kernel draw, whose tile sums live in the workspace:
    # 127 * ceil(V / 64) floats exceed 16 MiB at V = 2^26 / 2. Nothing is
    # launched, so the pointers may be small stand-ins of the right dtype.
    B, G, V = 127, 1, 1 << 25
    lib = sv.load_library()
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    i = torch.zeros(16, dtype=torch.int32, device="cuda")
    f = torch.zeros(16, dtype=torch.float32, device="cuda")
    rc = lib.spec_verify_noalloc(B, G, V, sv.SPEC_BF16, None, x.data_ptr(), x.data_ptr(),
                                 i.data_ptr(), f.data_ptr(), 0, 0, i.data_ptr(), i.data_ptr())
    assert rc == sv.SPEC_ESCRATCH
    assert b"scratch" in sv.load_library().spec_verify_strerror(rc)
    rc = lib.spec_verify_noalloc(0, G, V, sv.SPEC_BF16, None, None, None, None, None, 0, 0,
                                 None, None)
    assert rc == sv.binding.SPEC_OK
