import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_addoption(parser):
    parser.addoption("--sa-lib", default=None,
                     help="load this build of libsketchattn instead of the in-tree one (sanitizer runs)")
    parser.addoption("--oracle-lib", default=None,
                     help="load this build of the C oracle instead of oracle/libsa_oracle.so (sanitizer runs)")


def pytest_sessionstart(session):
    sa_lib = session.config.getoption("--sa-lib")
    oracle_lib = session.config.getoption("--oracle-lib")
    if sa_lib:
        import sketch_attention_flashsa_amd as sa
        sa._lib = sa.load_library(sa_lib)
    if oracle_lib:
        import oracle
        oracle._lib = oracle.load(oracle_lib)
