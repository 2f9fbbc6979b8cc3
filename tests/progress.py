"""Progress lines of long GPU tests: printed, and appended to
gpurun_out/test_progress.log so that a run whose output pytest captures
still shows it is alive while the oracle works through a large model."""
import os
import sys
import time

_LOG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out", "test_progress.log")


def progress(msg: str) -> None:
    line = f"{time.strftime('%H:%M:%S')} {msg}"
    print(line, flush=True)
    try:
        os.makedirs(os.path.dirname(_LOG), exist_ok=True)
        with open(_LOG, "a") as f:
            f.write(line + "\n")
    except OSError as e:                  # a read-only tree: the printed line still goes out
        print(f"progress log not written: {e}", file=sys.stderr, flush=True)
