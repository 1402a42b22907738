"""Plants plausible mistakes in a temporary copy of the CPU oracle and checks
that the pins in test_oracle_pins.py catch every one of them (CPU only)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "gqa mapping i % Hkv": ("return (i * n_kv) // n_q", "return i % n_kv"),
    "rope sign": ("a * sin + b * cos", "-a * sin + b * cos"),
    "no 1/sqrt(hd) scale": ("s = (K[:, g, :] @ q[i]) / np.sqrt(F64(hd))", "s = (K[:, g, :] @ q[i])"),
    "window one key too wide": ("max(0, p - window + 1)", "max(0, p - window)"),
    "silu on the up half": ("return (silu(gate) * up)", "return (gate * silu(up))"),
    "ffn residual dropped": ("            x = x + self.ffn(l, x)\n", "            x = self.ffn(l, x)\n"),
    "eps outside the root": ("np.sqrt(ms + eps)", "np.sqrt(ms) + eps"),
    "rope frequency exponent": ("-2.0 * c / head_dim", "-1.0 * c / head_dim"),
    "causal mask off": ("m = j <= pos", "m = j >= 0"),
    "kv cache not rounded": ("return a.astype(np.float16).astype(F64) if kv_fp16 else a", "return a"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    for d in ("oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutants.py", "test_*gpu*"))
    src = (tmp_path / "oracle" / "decoder.py").read_text()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    (tmp_path / "oracle" / "decoder.py").write_text(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"no pin caught the mutant '{name}':\n{r.stdout[-2000:]}"
