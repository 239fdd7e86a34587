"""Child process of the cross-process test of the deterministic mode (not a
test module): runs the fused layer in deterministic mode on seeded inputs and
writes the routing, weights and output bits to an .npz file.

usage: python tests/det_child.py OUT.npz
"""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import moe_layer_align_amd as moe  # noqa: E402
from synth import MoEConfig, gen_logits, gen_weights, gen_x  # noqa: E402

CASES = [
    (MoEConfig("det_bf16", E=16, k=4, H=512, I=384, dtype="bf16", ms=(1,), logits="normal"), 70, None),
    (MoEConfig("det_fp8", E=64, k=8, H=1024, I=768, dtype="fp8", ms=(1,), logits="normal"), 1100, (0.013, 0.004)),
]


def main(path: str) -> int:
    dev = torch.device("cuda:0")
    out = {}
    for cfg, M, scales in CASES:
        w13, w2, s13, s2 = gen_weights(cfg, 61, device=dev)
        x = gen_x(cfg.H, M, 61, sub=M).to(dev)
        lg = gen_logits(cfg, M, 61, sub=M).to(dev)
        ids = torch.empty(M, cfg.k, dtype=torch.int32, device=dev)
        wts = torch.empty(M, cfg.k, dtype=torch.float32, device=dev)
        kw = {}
        if cfg.dtype == "fp8":
            t = lambda v: torch.tensor([v], dtype=torch.float32, device=dev)
            kw = dict(w13_scale=t(s13), w2_scale=t(s2), x_scale=t(scales[0]), h_scale=t(scales[1]))
        y = moe.fused_forward(x, lg, w13, w2, cfg.k, cfg.dtype, topk_ids=ids, topk_weights=wts, deterministic=True,
                              **kw)
        torch.cuda.synchronize()
        out[cfg.name + "_ids"] = ids.cpu().numpy()
        out[cfg.name + "_w"] = wts.cpu().numpy().view(np.uint32)
        out[cfg.name + "_y"] = y.view(torch.int16).cpu().numpy()
    np.savez(path, **out)
    print("det child wrote %s" % path, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
