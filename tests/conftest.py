import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size parity, minutes of host time")
    # progress lines of long parity tests go to the terminal as they happen,
    # past output capture (a run that prints nothing for minutes looks hung)
    import gpu_util
    gpu_util.CAPTURE = config.pluginmanager.getplugin("capturemanager")
