"""The parity gate shared by the GPU tests: a HIP result against the oracle's
fp64 values.

  * max-abs error within the dtype's tolerance (fp32 1e-4; bf16 storage with
    fp32 accumulation 2e-2);
  * normwise relative error ||got - ref||_2 / ||ref||_2 at most 1e-2, which
    a max-abs gate alone does not give where outputs are small (a decode or
    chunk row averages thousands of values, so its entries are ~1/sqrt(w)
    and one misplaced row of the window shifts them by a few per cent);
  * every value finite.
The error is printed as max-abs, as a multiple of the output's RMS, and
normwise, so a run's log shows how much margin each comparison had."""
import numpy as np

F32_TOL = 1e-4
BF16_TOL = 2e-2
REL_TOL = 1e-2


def tol_of(dtype) -> float:
    import torch

    return BF16_TOL if dtype == torch.bfloat16 else F32_TOL


def gate(got, ref, dtype, what: str, tol: float | None = None, rel_tol: float = REL_TOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    if tol is None:
        tol = tol_of(dtype)
    diff = got - ref
    err = float(np.max(np.abs(diff))) if diff.size else 0.0
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    rel = float(np.linalg.norm(diff) / (np.linalg.norm(ref) + 1e-300))
    print(f"{what}: max-abs {err:.3g} ({err / (rms + 1e-300):.3g} x output RMS {rms:.3g}), "
          f"normwise relative {rel:.3g}")
    assert err <= tol, f"{what}: max-abs {err:.3g} > {tol}"
    assert rel <= rel_tol, f"{what}: normwise relative {rel:.3g} > {rel_tol}"
    return err, rel
