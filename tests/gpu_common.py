"""Helpers shared by the GPU tests: upload a workload, run the library, compare with the oracle."""
import os

import numpy as np
import torch

import mla_latent_space_amd as mla

# Tolerances on out (float32 [b, s, h, 512]) and lse. bf16 cache: rel L2 <= 5e-3, max abs
# <= 2e-2, |d lse| <= 1e-3. fp8 cache: compared with the oracle on the same dequantised
# values, rel L2 <= 3e-2 (the stated fp8 bound). Its max abs and lse bounds follow from
# the arithmetic: the kernel dequantises each value once into bf16 (relative error
# <= 2^-8, the unit roundoff of an 8-bit significand), which moves a score by at most
# softmax_scale * 2^-8 * sum_c |q_c z_c| (about 1e-1 in the worst case and 6e-3 typical for
# these N(0,1) draws, whose per-value errors have random signs); lse moves by no more than
# the largest score error, so fp8 lse is held to 2e-2, about three times the typical
# perturbation. out = sum_u p_u z_u with sum_u p_u = 1, and both z_u (the dequantised value)
# and p_u are rounded once to bf16, so |d out_c| <= 2 * 2^-8 * max_u |z_uc| besides the
# score term; the latent values of these workloads stay below 5 in magnitude, which gives
# max abs <= 4e-2 (reached only by rows with a handful of visible keys).
BF16_TOL = dict(rel_l2=5e-3, max_abs=2e-2, lse=1e-3)
FP8_TOL = dict(rel_l2=3e-2, max_abs=4e-2, lse=2e-2)


class Dev:
    """A workload's arrays on the GPU."""

    def __init__(self, w, device="cuda"):
        self.w = w
        self.q = torch.from_numpy(w.q.view(np.int16)).to(device).view(torch.bfloat16)
        if w.kv_dtype == "bf16":
            self.kv = torch.from_numpy(w.kv.view(np.int16)).to(device).view(torch.bfloat16)
            self.scales = None
        else:
            self.kv = torch.from_numpy(w.kv).to(device)
            self.scales = torch.from_numpy(w.kv_scales).to(device)
        self.bt = torch.from_numpy(w.block_table).to(device)
        self.sl = torch.from_numpy(w.seqlens).to(device)

    def plan(self, num_workers=None):
        return mla.get_split_plan(self.sl, self.w.s_q, self.w.heads, self.w.causal, num_workers)

    def run(self, num_workers=None, plan=None):
        if plan is None:
            plan = self.plan(num_workers)
        out, lse = mla.decode_fwd(self.q, self.kv, self.bt, self.sl, self.w.scale, kv_scales=self.scales,
                                  causal=self.w.causal, plan=plan)
        torch.cuda.synchronize()
        return out, lse


def compare(out, lse, ref_out, ref_lse, tol, what=""):
    """Relative L2 and max abs over out, max |d lse| over finite lse; -inf must match."""
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    assert np.isfinite(out).all(), f"{what}: non-finite out"
    ninf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), ninf), f"{what}: -inf lse pattern differs"
    denom = np.linalg.norm(ref_out)
    rel = np.linalg.norm(out - ref_out) / (denom if denom > 0 else 1.0)
    mabs = float(np.max(np.abs(out - ref_out))) if out.size else 0.0
    dl = float(np.max(np.abs(lse[~ninf] - ref_lse[~ninf]))) if (~ninf).any() else 0.0
    msg = f"{what}: rel_l2={rel:.3e} max_abs={mabs:.3e} max_dlse={dl:.3e}"
    log = os.environ.get("MLA_PARITY_LOG")
    if log:   # margins of passing cases, for the record
        with open(log, "a") as f:
            f.write(msg + "\n")
    assert rel <= tol["rel_l2"] and mabs <= tol["max_abs"] and dl <= tol["lse"], msg
    return rel, mabs, dl


def fp8_rope_ramp(w, heads_aligned=16, q_val=64.0):
    """Scores that grow along the sequence by hundreds of log2 units, on an fp8 cache through
    its bf16 rope channels (bytes 512..639 of a row): heads 0..15 put q_val on the 64 rope
    channels of the query, and every cached rope channel rises by j / (t - 1) at token j."""
    def to_f32(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).float().numpy()

    def to_bits(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(
            torch.int16).numpy().view(np.uint16)

    q = to_f32(w.q)
    q[:, :, :heads_aligned, 512:] = q_val
    w.q = to_bits(q)
    rope = to_f32(np.ascontiguousarray(w.kv[..., 512:]).view(np.uint16))
    for b, t in enumerate(w.seqlens):
        for j in range(int(t)):
            rope[w.block_table[b, j // 64], j % 64, :] += 1.0 * j / max(1, int(t) - 1)
    w.kv[..., 512:] = to_bits(rope).view(np.uint8).reshape(w.kv[..., 512:].shape)
