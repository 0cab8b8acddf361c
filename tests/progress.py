"""Progress lines for the long GPU checks, written to the terminal past
pytest's output capture so that a run of several minutes reports as it goes."""
import contextlib
import sys
import time

capture_manager = None  # pytest's capture manager, set by conftest at configure time


def log(msg):
    line = f"[{time.strftime('%H:%M:%S')}] {msg}"
    ctx = (capture_manager.global_and_fixture_disabled() if capture_manager is not None
           else contextlib.nullcontext())
    with ctx:
        print(line, file=sys.stderr, flush=True)


def ticker(name, every=20.0):
    """An OracleModel.on_layer callback that logs at most every `every` s."""
    last = [time.time()]

    def tick(li):
        if time.time() - last[0] >= every:
            last[0] = time.time()
            log(f"{name}: oracle layer {li}")
    return tick
