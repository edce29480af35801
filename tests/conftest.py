import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
# tests/test_oracle_mutations.py points this at a copy of oracle/ with a planted
# mistake, so that the pins in tests/test_oracle.py run against the mutant.
_MUTANT = os.environ.get("AQLM_ORACLE_MUTANT_DIR")
if _MUTANT:
    sys.path.insert(0, _MUTANT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
