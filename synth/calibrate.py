"""Write synth/zipf_calibration.json: the Zipf exponent that gives each workload its target skew.

Run as ``python -m synth.calibrate``.  Uses only the generator (no method
code): bisection on the exponent with the routing noise fixed, then records
the exponent, the realised maxvio and the home-only load ratio (largest
per-rank load over S*K without replicas) at full shape.
"""
import json
import sys
import time

import synth


def main(names=None):
    cal = synth.load_calibration()
    for name, wl in synth.WORKLOADS.items():
        if names and name not in names:
            continue
        for target in wl.maxvio_targets:
            if target is None or target == 0.0:
                continue
            for placement in ("receiver0", "donor0"):
                key = f"{name}:{target:g}:{placement}"
                if key in cal:
                    continue
                t0 = time.time()
                s = synth.calibrate_zipf(wl.dims, target, wl.base_seed, placement)
                idx, _ = synth.routing(wl.dims, s, wl.base_seed, placement)
                cal[key] = {"zipf_s": s, "maxvio": synth.realised_maxvio(idx, wl.dims.E),
                            "home_load_ratio": synth.home_load_ratio(idx, wl.dims)}
                print(key, cal[key], f"{time.time() - t0:.1f}s", flush=True)
                with open(synth.CALIBRATION_FILE, "w") as f:
                    json.dump(cal, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:])
