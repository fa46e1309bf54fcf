"""Helpers shared by the GPU parity tests: upload generator inputs, run the
three libdblock entry points, bring results back to the host."""
import sys

import numpy as np
import torch

from block_wise_decoding_amd import dblock


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X (torch.cuda unavailable)"
    dblock.load_library()
    return torch.device("cuda:0")


def note(msg: str):
    """Print and flush, so a failing GPU step is named in the log."""
    print(msg, flush=True)
    sys.stdout.flush()


def bf16(arr: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)


def upload(inp: dict, dev) -> dict:
    out = {}
    for k, v in inp.items():
        if k in ("q", "kp", "vp", "kb", "vb", "ks", "vs", "w", "h"):
            out[k] = bf16(v, dev)
        elif k in ("prefix_len", "tokens"):
            out[k] = torch.from_numpy(np.ascontiguousarray(v, dtype=np.int32)).to(dev)
        elif k == "mask":
            out[k] = torch.from_numpy(np.ascontiguousarray(v, dtype=np.uint8)).to(dev)
    return out


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> float64 numpy (exact)."""
    return t.float().cpu().numpy().astype(np.float64)


def run_attend(d: dict, scale: float = 0.0) -> torch.Tensor:
    B, L, H, D = d["q"].shape
    out = torch.empty_like(d["q"])
    dblock.dblk_attend(d["q"], d["kp"], d["vp"], d["kb"], d["vb"], d["ks"], d["vs"],
                       d.get("prefix_len"), out, scale=scale)
    return out


def run_lmhead(d: dict):
    M = d["h"].shape[0]
    conf = torch.empty(M, dtype=torch.float32, device=d["h"].device)
    amax = torch.empty(M, dtype=torch.int32, device=d["h"].device)
    dblock.dblk_lmhead_confidence(d["h"], d["w"], conf, amax)
    return conf, amax


def run_iteration(d: dict, tau: float):
    """attend + lmhead + commit on one stream; returns host numpy results."""
    o = run_attend(d)
    conf, amax = run_lmhead(d)
    B, L = d["tokens"].shape
    tok = d["tokens"].clone()
    msk = d["mask"].clone()
    n = torch.empty(B, dtype=torch.int32, device=tok.device)
    dblock.dblk_threshold_commit(conf.view(B, L), amax.view(B, L), tok, msk, tau, n)
    torch.cuda.synchronize()
    return {"o": bf16_to_np(o), "conf": conf.cpu().numpy(), "argmax": amax.cpu().numpy(),
            "tokens": tok.cpu().numpy(), "mask": msk.cpu().numpy(), "n": n.cpu().numpy()}
