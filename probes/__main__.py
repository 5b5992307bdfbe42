"""``python -m probes``: build the measurement probes."""
from probes import build

print(build(verbose=True))
