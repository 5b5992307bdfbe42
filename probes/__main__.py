"""``python -m probes``: build the measurement probes.
``python -m probes timeline [--out FILE]``: run the timeline probe (GPU)."""
import sys

if len(sys.argv) > 1 and sys.argv[1] == "timeline":
    from probes import timeline
    out = sys.argv[sys.argv.index("--out") + 1] if "--out" in sys.argv else None
    timeline.main(out)
else:
    from probes import build
    print(build(verbose=True))
