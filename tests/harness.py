"""Test-side names for the oracle driver (oracle/drive.py)."""
from oracle.drive import OracleStep, oracle_cfg  # noqa: F401
