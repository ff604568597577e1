"""CPU oracle (test infrastructure only; see ``lora_oracle`` for the rules)."""
from .lora_oracle import *  # noqa: F401,F403
from . import lora_oracle  # noqa: F401
