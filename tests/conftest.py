import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large-workload checks (minutes)")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Parity counts of this session (CSR rows exact / excused (A) / near-tie (B) / failed, and the
    attention errors), one line per checked case, so that a -q run's tail carries them."""
    try:
        from _parity import RECORDS
    except Exception:  # pragma: no cover
        return
    if not RECORDS:
        return
    tr = terminalreporter
    tr.section("parity records")
    keys = ("rows", "exact", "excused_A", "neartie_B", "fail", "kept_frac", "attn_rows", "attn_max_abs",
            "attn_mean_abs", "bf16_max_abs", "bf16_mean_abs", "bf16_max_abs_beyond_rounding", "bf16_mean_abs_beyond_rounding", "max_abs", "mean_abs", "status")
    tot = dict(rows=0, exact=0, excused_A=0, neartie_B=0, fail=0)
    for name, pl in RECORDS:
        if "exact" in pl and "rows" in pl:
            for k in tot:
                tot[k] += int(pl.get(k, 0))
        if "/full" not in name and not name.startswith("full/"):
            continue      # small cases: counted in the totals only
        parts = []
        for k in keys:
            if k in pl:
                v = pl[k]
                parts.append(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}")
        tr.write_line(f"{name}: " + " ".join(parts))
    tr.write_line("CSR rows checked: " + " ".join(f"{k}={v}" for k, v in tot.items()))
