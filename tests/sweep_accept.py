"""Oracle check of the offline tile sweep's forward variants (GPU).

    python tests/sweep_accept.py [--dims 64,128] > accepted.jsonl

Every variant library built by `python -m exact_attention_121_amd.tile_sweep
build` runs the validation problems of its head_dim -- a ragged sequence
length with GQA and spiky logits (1 % of Q and K rows x8), causal and not,
and a longer non-causal MHA head pair -- and is compared with the fp64 oracle
at the parity bar (max |dO| <= 1e-2, mean |dO| <= 1e-3, |dLSE| <= 1e-3, no
NaN/Inf).  One JSON line per variant: {"variant", "accepted", "cases": [...]};
`tile_sweep run --accepted` times only the accepted ones.  Test
infrastructure: the package itself never calls the oracle.
"""

import argparse
import json
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402,F401  (torch's HIP runtime first, then the variant libraries)

from exact_attention_121_amd import tile_sweep  # noqa: E402
from exact_attention_121_amd.inputs import make_qkv  # noqa: E402
from oracle.attention import attention_ref  # noqa: E402

BAR = (1e-2, 1e-3, 1e-3)


def problems(d):
    """(B, Hq, Hkv, N, causal, spike_frac, seed) validation problems of head_dim d."""
    return [(1, 4, 2, 777, False, 0.01, 11 + d), (1, 4, 2, 777, True, 0.01, 12 + d),
            (1, 2, 2, 2048, False, 0.0, 13 + d), (2, 2, 1, 300, True, 0.0, 14 + d)]


def check(lib, d, prob, refs):
    import torch

    B, Hq, Hkv, N, causal, spikes, seed = prob
    qn, kn, vn = make_qkv(B, Hq, Hkv, N, d, seed=seed, spike_frac=spikes, spike_mult=8.0)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    key = (d, prob)
    if key not in refs:
        refs[key] = attention_ref(qn, kn, vn, scale, causal=causal)
    O_ref, L_ref = refs[key]
    q, k, v = (torch.from_numpy(x).cuda() for x in (qn, kn, vn))
    o, lse = torch.empty_like(q), torch.empty(B, Hq, N, device="cuda")
    st = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d,
                      scale, int(causal), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    if st != 0:
        return {"problem": prob, "ok": False, "status": st}
    og = o.cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    finite = bool(np.isfinite(og).all() and np.isfinite(lg).all())
    err = np.abs(og - O_ref)
    lerr = np.abs(lg - L_ref)
    ok = finite and err.max() <= BAR[0] and err.mean() <= BAR[1] and lerr.max() <= BAR[2]
    return {"problem": prob, "ok": bool(ok), "max_abs_err_O": float(err.max()), "mean_abs_err_O": float(err.mean()),
            "max_abs_err_LSE": float(lerr.max())}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--dims", default="")
    args = ap.parse_args()
    dims = {int(x) for x in args.dims.split(",")} if args.dims else None
    refs = {}
    for d, vdef, name in tile_sweep.all_variants(dims):
        path = tile_sweep.variant_path(name)
        if not os.path.exists(path):
            print(json.dumps({"variant": name, "accepted": False, "reason": "not built"}), flush=True)
            continue
        lib = tile_sweep.load_variant(path)
        cases = [check(lib, d, prob, refs) for prob in problems(d)]
        print(json.dumps({"variant": name, "accepted": all(c["ok"] for c in cases), "cases": cases}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
