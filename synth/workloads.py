"""Workload shapes for the NABLA hot path.

Each workload is a synthetic stand-in for a setting the NABLA paper measures
("NABLA: Neighborhood Adaptive Block-Level Attention", section 4.1 fine-tuning of
Wan 2.1 14B at 720p, and section 4.3 pretraining of a 2B DiT at 512x512). None of
the paper's weights, activations or prompts are used; the inputs only take the
shapes of those settings and the spatio-temporal locality the paper's Appendix D
(Figure 9) shows in real attention maps.

The input scale ``alpha`` and the CDF thresholds of the bf16 workloads are
calibrated with the CPU oracle by ``oracle/calibrate.py`` and stored in
``synth/calibration.json``; this module only reads them.
"""

from __future__ import annotations

import json
import os
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

_CALIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "calibration.json")


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    T: int          # latent frames
    Hs: int         # latent height in tokens
    Ws: int         # latent width in tokens
    P: int = 8      # spatial tile edge; block size N = P*P
    dtype: str = "bf16"          # "fp32": Q/K/V kept as fp32 (rounded to bf16 at the GPU boundary)
    noise_std: float = 0.5       # std of the per-tensor noise added to the shared field
    shared_v: bool = False       # V = F + noise (True) or V ~ N(0,1) (False)
    scaled: bool = True          # Q, K multiplied by a calibrated alpha
    # How alpha is calibrated: "table1" -- thr = 0.7 gives 80.13% block sparsity,
    # the NABLA(0.7) row of the paper's Table 1; "std3" -- the pooled logits
    # Q_a . K_a / sqrt(D) have a standard deviation of 3.
    alpha_rule: str = "table1"
    target_sparsity: Tuple[float, ...] = ()
    fixed_thr: Tuple[float, ...] = ()
    sta: Optional[Tuple[int, int, int]] = None   # (win_t, win_h, win_w) in tokens
    thr_from: Optional[str] = None               # reuse another workload's alpha and thr
    backward: bool = False
    seed_base: int = 0
    description: str = ""

    @property
    def N(self) -> int:
        return self.P * self.P

    @property
    def S(self) -> int:
        return self.T * self.Hs * self.Ws

    @property
    def n(self) -> int:
        return self.S // self.N

    def seed(self, step: int = 0) -> int:
        return 1000 * self.seed_base + step

    def sta_struct(self) -> Optional[Dict[str, int]]:
        if self.sta is None:
            return None
        return dict(T=self.T, Hs=self.Hs, Ws=self.Ws, P=self.P,
                    win_t=self.sta[0], win_h=self.sta[1], win_w=self.sta[2])

    def calibration(self) -> Dict:
        key = self.thr_from or self.name
        data = load_calibration()
        base = dict(data.get(self.name, {}))
        if self.thr_from:
            other = data.get(key, {})
            base.setdefault("thr", other.get("thr", {}))
        return base

    def alpha(self) -> float:
        if not self.scaled:
            return 1.0
        cal = load_calibration().get(self.thr_from or self.name)
        if cal is None or "alpha" not in cal:
            raise KeyError(f"workload {self.name}: alpha not calibrated; run oracle/calibrate.py")
        return float(cal["alpha"])

    def thresholds(self) -> List[float]:
        """CDF thresholds to run: fixed ones, else the calibrated ones (per target)."""
        if self.fixed_thr:
            return list(self.fixed_thr)
        cal = self.calibration()
        thr = cal.get("thr", {})
        if not thr:
            raise KeyError(f"workload {self.name}: thresholds not calibrated; run oracle/calibrate.py")
        return [float(thr[k]) for k in sorted(thr)]

    def thr_for(self, sparsity: float) -> float:
        thr = self.calibration().get("thr", {})
        key = f"{sparsity:.2f}"
        if key not in thr:
            raise KeyError(f"workload {self.name}: no calibrated thr for sparsity {key}")
        return float(thr[key])


def load_calibration() -> Dict:
    if not os.path.exists(_CALIB_PATH):
        return {}
    with open(_CALIB_PATH) as f:
        return json.load(f)


WORKLOADS: Dict[str, Workload] = {
    # B=1, H=2, D=64, 4 frames of 16x16 tokens, 8x8 tiles -> 16 blocks of 64.
    "tiny": Workload(
        name="tiny", B=1, H=2, D=64, T=4, Hs=16, Ws=16, dtype="fp32", noise_std=1.0,
        shared_v=True, scaled=False, fixed_thr=(0.2, 0.5, 0.9, 1.0), seed_base=1,
        description="B1 H2 D64, latent 4x16x16 = 1024 tokens (16 blocks), fp32, thr sweep"),
    # B=1, H=12, D=128, 11x32x32 = 11264 tokens (176 blocks).
    "dit_small": Workload(
        name="dit_small", B=1, H=12, D=128, T=11, Hs=32, Ws=32, target_sparsity=(0.80,),
        seed_base=2,
        description="B1 H12 D128, latent 11x32x32 = 11264 tokens (176 blocks), ~80% sparse"),
    # Wan 2.1 14B-like layer at 720p: B=1, H=40, D=128, 21x48x80 = 80640 tokens (1260 blocks).
    "wan14b_720p": Workload(
        name="wan14b_720p", B=1, H=40, D=128, T=21, Hs=48, Ws=80,
        target_sparsity=(0.80, 0.90), seed_base=3,
        description="B1 H40 D128, latent 21x48x80 = 80640 tokens (1260 blocks), 80% and 90% sparse"),
    # dit_small shape with the NABLA mask unioned with an STA window of 11 frames x 3x3 tiles.
    "dit_small_sta": Workload(
        name="dit_small_sta", B=1, H=12, D=128, T=11, Hs=32, Ws=32, sta=(11, 24, 24),
        thr_from="dit_small", seed_base=2,
        description="dit_small inputs, NABLA(thr of dit_small) OR STA(11,24,24)"),
    # dit_small shape with alpha set so the pooled logits have std 3 (very peaked rows).
    "dit_small_std3": Workload(
        name="dit_small_std3", B=1, H=12, D=128, T=11, Hs=32, Ws=32, target_sparsity=(0.80,),
        alpha_rule="std3", seed_base=2,
        description="dit_small inputs scaled to pooled-logit std 3, ~80% sparse"),
    # The 720p layer on the literal recipe: alpha set so the pooled logits have std 3.
    "wan14b_720p_std3": Workload(
        name="wan14b_720p_std3", B=1, H=40, D=128, T=21, Hs=48, Ws=80,
        target_sparsity=(0.80, 0.90), alpha_rule="std3", seed_base=3,
        description="wan14b_720p inputs scaled to pooled-logit std 3, 80% and 90% sparse"),
    # 2B video DiT training shape: B=2, H=16, D=128, 16x48x80 = 61440 tokens (960 blocks).
    "dit2b_train": Workload(
        name="dit2b_train", B=2, H=16, D=128, T=16, Hs=48, Ws=80, target_sparsity=(0.85,),
        backward=True, seed_base=5,
        description="B2 H16 D128, latent 16x48x80 = 61440 tokens (960 blocks), ~85% sparse, fwd+bwd"),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]
